"""Thin ctypes binding of ``libfrt.so`` (the C ABI in ``include/frt.h``).

Argument marshalling only: torch tensors are passed as device pointers, the current
torch stream as the hipStream_t, and a non-zero status raises ``FrtError``.  Every step
of the computation runs in the library's HIP kernels; there is no fallback.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; FRT_LIBRARY names another build of the same sources (the host-side
# sanitizer build of the CPU tests)
LIB_PATH = os.environ.get("FRT_LIBRARY") or os.path.join(_HERE, "libfrt.so")

OK, E_NULL, E_SHAPE, E_ALIGN, E_DTYPE, E_SPLITK, E_WORKSPACE, E_ALIAS, E_STATE, E_HIP, E_ARG = range(11)
BF16, E4M3, F32, MXFP4 = 1, 2, 3, 4
W_PLAIN, W_GATE_UP = 0, 1
EPI_NONE, EPI_STORE_F32, EPI_STORE_BF16, EPI_SILU_GATE_QUANT = 0, 1, 2, 3
DTYPES = {"bf16": BF16, "e4m3": E4M3, "f32": F32, "mxfp4": MXFP4}


def act_dtype(wdtype):
    """GEMM operand format that goes with a weight format (MXFP4 weights take e4m3)."""
    return E4M3 if wdtype == MXFP4 else wdtype

_c_void_p = ctypes.c_void_p
_int = ctypes.c_int
_float = ctypes.c_float
_size = ctypes.c_size_t


class FrtError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = _lib().frt_status_string(status).decode()
        if status == E_HIP:
            msg += f" (hipError {_lib().frt_last_hip_error()})"
        super().__init__(f"{where}: status {status}: {msg}")


class ChainDesc(ctypes.Structure):
    _fields_ = [("layers", _int), ("steps", _int), ("M", _int), ("hidden", _int), ("n_heads", _int),
                ("head_dim", _int), ("prefix_len", _int), ("mlp", _int), ("dtype", _int), ("eps", _float),
                ("splits_qkv", _int), ("splits_o", _int), ("splits_up", _int), ("splits_down", _int),
                ("use_graph", _int), ("keep_intermediates", _int), ("prefetch_next", _int),
                ("w_qkv", ctypes.POINTER(_c_void_p)), ("w_o", ctypes.POINTER(_c_void_p)),
                ("w_up", ctypes.POINTER(_c_void_p)), ("w_down", ctypes.POINTER(_c_void_p)),
                ("s_qkv", ctypes.POINTER(_c_void_p)), ("s_o", ctypes.POINTER(_c_void_p)),
                ("s_up", ctypes.POINTER(_c_void_p)), ("s_down", ctypes.POINTER(_c_void_p))]


_SIGS = {
    "frt_status_string": (ctypes.c_char_p, [_int]),
    "frt_last_hip_error": (_int, []),
    "frt_version": (_int, []),
    "frt_diag_empty_kernels": (_int, [_c_void_p, _int, _int]),
    "frt_operand_bytes": (_size, [_int, _int, _int]),
    "frt_weight_bytes": (_size, [_int, _int, _int]),
    "frt_operand_pack_host": (_int, [_c_void_p, _int, _int, _int, _c_void_p]),
    "frt_operand_unpack_host": (_int, [_c_void_p, _int, _int, _int, _c_void_p]),
    "frt_weight_pack_host": (_int, [_c_void_p, _int, _int, _int, _int, _c_void_p]),
    "frt_weight_unpack_host": (_int, [_c_void_p, _int, _int, _int, _int, _c_void_p]),
    "frt_weight_pack_mxfp4_host": (_int, [_c_void_p, _c_void_p, _int, _int, _int, _c_void_p]),
    "frt_weight_unpack_mxfp4_host": (_int, [_c_void_p, _int, _int, _int, _c_void_p, _c_void_p]),
    "frt_pack_weight": (_int, [_c_void_p, _int, _int, _c_void_p, _c_void_p, _int, _int, _c_void_p, _c_void_p]),
    "frt_residual_norm_quant": (_int, [_c_void_p, _int, _int, _c_void_p, _int, _float, _c_void_p, _c_void_p,
                                       _c_void_p, _c_void_p, _c_void_p, _c_void_p, _float, _int, _float,
                                       _c_void_p]),
    "frt_skinny_gemm_splitk": (_int, [_c_void_p, _int, _int, _int, _int, _int, _int, _c_void_p, _c_void_p,
                                      _c_void_p, _float, _c_void_p, _size, _int, _c_void_p, _int, _float]),
    "frt_skinny_gemm_splitk_noalloc": (_int, [_c_void_p, _int, _int, _int, _int, _int, _int, _c_void_p, _c_void_p,
                                              _c_void_p, _float, _int, _c_void_p, _int, _float]),
    "frt_noalloc_scratch_bytes": (_size, []),
    "frt_splitk_reduce": (_int, [_c_void_p, _int, _int, _int, _c_void_p, _float, _c_void_p, _int, _c_void_p,
                                 _int, _float]),
    "frt_splitk_choose": (_int, [_int, _int, _int, _int]),
    "frt_skinny_gemm_qkv": (_int, [_c_void_p, _int, _int, _int, _int, _int, _int, _c_void_p, _c_void_p, _c_void_p,
                                   _float, _c_void_p, _size, _c_void_p, _c_void_p, _c_void_p, _int]),
    "frt_attention_workspace_bytes": (_size, [_int, _int, _int, _int]),
    "frt_attention_prefix": (_int, [_c_void_p, _int, _int, _int, _int, _c_void_p, _c_void_p, _c_void_p, _int,
                                    _int, _float, _c_void_p, _c_void_p, _size]),
    "frt_layer_chain_arena_bytes": (_size, [ctypes.POINTER(ChainDesc)]),
    "frt_layer_chain_create": (_int, [ctypes.POINTER(ChainDesc), _c_void_p, _size, _c_void_p,
                                      ctypes.POINTER(_c_void_p)]),
    "frt_layer_chain_buffer": (_int, [_c_void_p, ctypes.c_char_p, ctypes.POINTER(_c_void_p),
                                      ctypes.POINTER(_size)]),
    "frt_layer_chain_run": (_int, [_c_void_p, _c_void_p]),
    "frt_layer_chain_calibrate": (_int, [_c_void_p, _c_void_p, _c_void_p]),
    "frt_layer_chain_kernel_count": (_int, [_c_void_p]),
    "frt_layer_chain_state_bytes": (_size, [_c_void_p]),
    "frt_layer_chain_snapshot": (_int, [_c_void_p, _c_void_p, _c_void_p, _size]),
    "frt_layer_chain_restore": (_int, [_c_void_p, _c_void_p, _c_void_p, _size]),
    "frt_layer_chain_destroy": (_int, [_c_void_p]),
}

_LIB = None


def _lib():
    """Load libfrt.so (built in-tree by ``gemm_chains_amd.build``); fail loudly if absent."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                               "(run python -c 'import __graft_entry__ as g; g.build()')")
        # torch ships its own HIP runtime under the same soname as the system one that the
        # library links; whichever loads first serves the whole process, and torch needs
        # its own, so torch is imported before the library is loaded
        import torch  # noqa: F401
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def lib():
    return _lib()


def _ptr(t):
    """Device pointer of a tensor (or None/int passthrough)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status, where):
    if status != OK:
        raise FrtError(status, where)


def frt_diag_empty_kernels(n, workgroups, stream=None):
    _check(_lib().frt_diag_empty_kernels(_stream(stream), n, workgroups), "frt_diag_empty_kernels")


# ------------------------------------------------------------------ layout helpers

def frt_operand_bytes(dtype, M, K):
    return _lib().frt_operand_bytes(dtype, M, K)


def frt_weight_bytes(dtype, K, N):
    return _lib().frt_weight_bytes(dtype, K, N)


def frt_splitk_choose(M, N, K, dtype):
    return _lib().frt_splitk_choose(M, N, K, dtype)


def _np_ptr(a):
    return a.ctypes.data_as(_c_void_p)


def frt_operand_pack_host(codes, dtype, M, K):
    """numpy codes [M][K] (uint16 bf16 / uint8 e4m3) -> packed bytes (numpy uint8)."""
    import numpy as np
    codes = np.ascontiguousarray(codes)
    out = np.zeros(frt_operand_bytes(dtype, M, K), np.uint8)
    _check(_lib().frt_operand_pack_host(_np_ptr(codes), dtype, M, K, _np_ptr(out)), "frt_operand_pack_host")
    return out


def frt_operand_unpack_host(packed, dtype, M, K):
    import numpy as np
    packed = np.ascontiguousarray(packed).view(np.uint8)
    out = np.zeros((M, K), np.uint16 if dtype == BF16 else np.uint8)
    _check(_lib().frt_operand_unpack_host(_np_ptr(packed), dtype, M, K, _np_ptr(out)), "frt_operand_unpack_host")
    return out


def frt_weight_pack_host(codes, dtype, K, N, layout=W_PLAIN):
    import numpy as np
    codes = np.ascontiguousarray(codes)
    out = np.zeros(frt_weight_bytes(dtype, K, N), np.uint8)
    _check(_lib().frt_weight_pack_host(_np_ptr(codes), dtype, K, N, layout, _np_ptr(out)), "frt_weight_pack_host")
    return out


def frt_weight_unpack_host(packed, dtype, K, N, layout=W_PLAIN):
    import numpy as np
    packed = np.ascontiguousarray(packed).view(np.uint8)
    out = np.zeros((K, N), np.uint16 if dtype == BF16 else np.uint8)
    _check(_lib().frt_weight_unpack_host(_np_ptr(packed), dtype, K, N, layout, _np_ptr(out)),
           "frt_weight_unpack_host")
    return out


def frt_weight_pack_mxfp4_host(codes, scales, K, N, layout=W_PLAIN):
    """codes [K][N] FP4 codes (uint8, low 4 bits), scales [K/32][N] E8M0 bytes -> packed bytes."""
    import numpy as np
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    out = np.zeros(frt_weight_bytes(MXFP4, K, N), np.uint8)
    _check(_lib().frt_weight_pack_mxfp4_host(_np_ptr(codes), _np_ptr(scales), K, N, layout, _np_ptr(out)),
           "frt_weight_pack_mxfp4_host")
    return out


def frt_weight_unpack_mxfp4_host(packed, K, N, layout=W_PLAIN):
    """Packed MXFP4 bytes -> (codes [K][N], scale bytes [K/32][N])."""
    import numpy as np
    packed = np.ascontiguousarray(packed).view(np.uint8)
    codes = np.zeros((K, N), np.uint8)
    scales = np.zeros((K // 32, N), np.uint8)
    _check(_lib().frt_weight_unpack_mxfp4_host(_np_ptr(packed), K, N, layout, _np_ptr(codes), _np_ptr(scales)),
           "frt_weight_unpack_mxfp4_host")
    return codes, scales


# ------------------------------------------------------------------ device entry points

def frt_pack_weight(K, N, w_bf16, gamma, dtype, layout, w_packed, colscale, stream=None):
    _check(_lib().frt_pack_weight(_stream(stream), K, N, _ptr(w_bf16), _ptr(gamma), dtype, layout, _ptr(w_packed),
                                  _ptr(colscale)), "frt_pack_weight")


def frt_residual_norm_quant(M, K, x, x_splits, x_scale, x_colscale, residual, residual_out, gate, ada_scale,
                            ada_shift, eps, out_dtype, act_scale, operand_out, stream=None):
    _check(_lib().frt_residual_norm_quant(_stream(stream), M, K, _ptr(x), x_splits, x_scale, _ptr(x_colscale),
                                          _ptr(residual), _ptr(residual_out), _ptr(gate), _ptr(ada_scale),
                                          _ptr(ada_shift), eps, out_dtype, act_scale, _ptr(operand_out)),
           "frt_residual_norm_quant")


def frt_skinny_gemm_splitk(M, N, K, splits, ab_dtype, layout, a_packed, w_packed, w_colscale, act_scale, partials,
                           partials_bytes, epi, out, out_dtype, out_act_scale, stream=None):
    _check(_lib().frt_skinny_gemm_splitk(_stream(stream), M, N, K, splits, ab_dtype, layout, _ptr(a_packed),
                                         _ptr(w_packed), _ptr(w_colscale), act_scale, _ptr(partials),
                                         partials_bytes, epi, _ptr(out), out_dtype, out_act_scale),
           "frt_skinny_gemm_splitk")


def frt_skinny_gemm_splitk_noalloc(M, N, K, splits, ab_dtype, layout, a_packed, w_packed, w_colscale, act_scale, epi,
                                   out, out_dtype, out_act_scale, stream=None):
    _check(_lib().frt_skinny_gemm_splitk_noalloc(_stream(stream), M, N, K, splits, ab_dtype, layout, _ptr(a_packed),
                                                 _ptr(w_packed), _ptr(w_colscale), act_scale, epi, _ptr(out),
                                                 out_dtype, out_act_scale), "frt_skinny_gemm_splitk_noalloc")


def frt_noalloc_scratch_bytes():
    return _lib().frt_noalloc_scratch_bytes()


def frt_splitk_reduce(M, N, splits, partials, act_scale, w_colscale, epi, out, out_dtype, out_act_scale,
                      stream=None):
    _check(_lib().frt_splitk_reduce(_stream(stream), M, N, splits, _ptr(partials), act_scale, _ptr(w_colscale),
                                    epi, _ptr(out), out_dtype, out_act_scale), "frt_splitk_reduce")


def frt_skinny_gemm_qkv(M, K, n_heads, head_dim, splits, ab_dtype, a_packed, w_packed, w_colscale, act_scale,
                        partials, partials_bytes, q_out, k_out, v_t_out, v_ld, stream=None):
    _check(_lib().frt_skinny_gemm_qkv(_stream(stream), M, K, n_heads, head_dim, splits, ab_dtype, _ptr(a_packed),
                                      _ptr(w_packed), _ptr(w_colscale), act_scale, _ptr(partials), partials_bytes,
                                      _ptr(q_out), _ptr(k_out), _ptr(v_t_out), v_ld), "frt_skinny_gemm_qkv")


def frt_attention_workspace_bytes(M, n_heads, head_dim, kv_len):
    return _lib().frt_attention_workspace_bytes(M, n_heads, head_dim, kv_len)


def frt_attention_prefix(M, n_heads, head_dim, kv_len, q, k, v_t, ldv, out_dtype, out_act_scale, operand_out,
                         workspace, workspace_bytes, stream=None):
    _check(_lib().frt_attention_prefix(_stream(stream), M, n_heads, head_dim, kv_len, _ptr(q), _ptr(k), _ptr(v_t),
                                       ldv, out_dtype, out_act_scale, _ptr(operand_out), _ptr(workspace),
                                       workspace_bytes), "frt_attention_prefix")


# ------------------------------------------------------------------ chain

def _ptr_array(ptrs):
    arr = (_c_void_p * len(ptrs))(*[_ptr(p) for p in ptrs])
    return arr, ctypes.cast(arr, ctypes.POINTER(_c_void_p))


def make_chain_desc(layers, steps, M, hidden, n_heads, head_dim, prefix_len, mlp, dtype, eps, splits,
                    w_qkv, w_o, w_up, w_down, s_qkv=None, s_o=None, s_up=None, s_down=None, use_graph=True,
                    keep_intermediates=False, prefetch_next=False):
    """Build a ChainDesc; returns (desc, keepalive) -- keep both alive while the chain exists."""
    keep = []
    d = ChainDesc()
    d.layers, d.steps, d.M, d.hidden = layers, steps, M, hidden
    d.n_heads, d.head_dim, d.prefix_len, d.mlp = n_heads, head_dim, prefix_len, mlp
    d.dtype, d.eps = dtype, eps
    d.splits_qkv, d.splits_o, d.splits_up, d.splits_down = splits
    d.use_graph, d.keep_intermediates = int(bool(use_graph)), int(bool(keep_intermediates))
    d.prefetch_next = int(bool(prefetch_next))
    for name, ptrs in (("w_qkv", w_qkv), ("w_o", w_o), ("w_up", w_up), ("w_down", w_down),
                       ("s_qkv", s_qkv), ("s_o", s_o), ("s_up", s_up), ("s_down", s_down)):
        if ptrs is None:
            setattr(d, name, None)
            continue
        arr, p = _ptr_array(ptrs)
        keep.append(arr)
        setattr(d, name, p)
    return d, keep


def frt_layer_chain_arena_bytes(desc):
    return _lib().frt_layer_chain_arena_bytes(ctypes.byref(desc))


def frt_layer_chain_create(desc, arena, arena_bytes, capture_stream=None):
    h = _c_void_p()
    _check(_lib().frt_layer_chain_create(ctypes.byref(desc), _ptr(arena), arena_bytes, _stream(capture_stream),
                                         ctypes.byref(h)), "frt_layer_chain_create")
    return h


def frt_layer_chain_buffer(chain, name):
    dev = _c_void_p()
    nbytes = _size()
    _check(_lib().frt_layer_chain_buffer(chain, name.encode(), ctypes.byref(dev), ctypes.byref(nbytes)),
           f"frt_layer_chain_buffer({name})")
    return dev.value, nbytes.value


def frt_layer_chain_run(chain, stream=None):
    _check(_lib().frt_layer_chain_run(chain, _stream(stream)), "frt_layer_chain_run")


def frt_layer_chain_calibrate(chain, scales, stream=None):
    _check(_lib().frt_layer_chain_calibrate(chain, _stream(stream), _ptr(scales)), "frt_layer_chain_calibrate")


def frt_layer_chain_kernel_count(chain):
    return _lib().frt_layer_chain_kernel_count(chain)


def frt_layer_chain_state_bytes(chain):
    return _lib().frt_layer_chain_state_bytes(chain)


def frt_layer_chain_snapshot(chain, capsule, capsule_bytes, stream=None):
    _check(_lib().frt_layer_chain_snapshot(chain, _stream(stream), _ptr(capsule), capsule_bytes),
           "frt_layer_chain_snapshot")


def frt_layer_chain_restore(chain, capsule, capsule_bytes, stream=None):
    _check(_lib().frt_layer_chain_restore(chain, _stream(stream), _ptr(capsule), capsule_bytes),
           "frt_layer_chain_restore")


def frt_layer_chain_destroy(chain):
    _check(_lib().frt_layer_chain_destroy(chain), "frt_layer_chain_destroy")
