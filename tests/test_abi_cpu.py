"""C ABI checks that need no GPU: the library loads, exports every declared symbol,
validates arguments before any HIP call, and its host layout helpers are bijections.

Calls with made-up device pointers are only made where validation must reject them; they
are skipped when a GPU is visible, so a made-up pointer can never reach a kernel.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from gemm_chains_amd import frt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "frt.h")


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


no_gpu = pytest.mark.skipif(_gpu_visible(), reason="made-up device pointers are only passed where no GPU exists")

FAKE = 0x7f0000000000  # 16-byte aligned, never dereferenced (validation rejects first)


def test_library_loads_and_exports_every_declared_symbol():
    lib = frt.lib()
    text = open(HEADER).read()
    names = sorted(set(re.findall(r"\b(frt_[a-z0-9_]+)\s*\(", text)))
    assert len(names) >= 20
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert lib.frt_version() == 100
    for st in range(11):
        assert lib.frt_status_string(st)
    assert lib.frt_last_hip_error() == 0


def test_sizes_and_split_table():
    assert frt.frt_operand_bytes(frt.BF16, 10, 1024) == 16 * 1024 * 2
    assert frt.frt_operand_bytes(frt.E4M3, 50, 1024) == 64 * 1024
    assert frt.frt_operand_bytes(frt.BF16, 65, 1024) == 0
    assert frt.frt_weight_bytes(frt.E4M3, 1024, 8192) == 1024 * 8192
    assert frt.frt_weight_bytes(frt.BF16, 4096, 1024) == 4096 * 1024 * 2
    for (M, N, K, dt) in [(10, 1024, 1024, frt.BF16), (50, 8192, 1024, frt.BF16), (50, 1024, 4096, frt.BF16),
                          (10, 2560, 1024, frt.E4M3), (64, 16384, 2048, frt.E4M3)]:
        s = frt.frt_splitk_choose(M, N, K, dt)
        kst = K // (32 if dt == frt.BF16 else 128)
        assert s in (1, 2, 4, 8, 16) and kst % s == 0
    assert frt.frt_splitk_choose(0, 1024, 1024, frt.BF16) == 0
    assert frt.frt_splitk_choose(10, 1000, 1024, frt.BF16) == 0


@pytest.mark.parametrize("dtype,M,K", [(frt.BF16, 10, 1024), (frt.BF16, 17, 96), (frt.E4M3, 50, 1024),
                                       (frt.E4M3, 64, 128), (frt.BF16, 1, 32)])
def test_operand_layout_is_a_bijection(dtype, M, K):
    g = np.random.default_rng(M + K)
    codes = g.integers(0, 1 << (16 if dtype == frt.BF16 else 8), (M, K)).astype(np.uint16 if dtype == frt.BF16 else np.uint8)
    packed = frt.frt_operand_pack_host(codes, dtype, M, K)
    assert packed.size == frt.frt_operand_bytes(dtype, M, K)
    assert np.array_equal(frt.frt_operand_unpack_host(packed, dtype, M, K), codes)
    # every element lands on its own bytes: packing an index pattern hits each slot once
    Mp = 16 * ((M + 15) // 16)
    idx = (np.arange(Mp * K).reshape(Mp, K) % (1 << 15) + 1).astype(np.uint16 if dtype == frt.BF16 else np.uint8)
    if dtype == frt.E4M3:
        idx = ((np.arange(Mp * K).reshape(Mp, K) % 255) + 1).astype(np.uint8)
    full = frt.frt_operand_pack_host(idx, dtype, Mp, K)
    assert np.count_nonzero(full.view(idx.dtype)) == Mp * K
    # padding rows are zero codes
    ppad = frt.frt_operand_unpack_host(packed, dtype, Mp, K)
    assert np.all(ppad[M:] == 0)


def test_operand_tile_structure_bf16():
    """One 16-byte lane slot = 8 consecutive k of one row; one 1 KB tile = 16 rows x 32 k."""
    M, K = 16, 64
    codes = (np.arange(M)[:, None] * 1000 + np.arange(K)[None, :]).astype(np.uint16)
    p = frt.frt_operand_pack_host(codes, frt.BF16, M, K).view(np.uint16)
    slot = p[:8]
    assert np.array_equal(slot, codes[0, :8])
    lane17 = p[17 * 8:18 * 8]                      # lane 17: row 1, k 8..15
    assert np.array_equal(lane17, codes[1, 8:16])
    tile1 = p[512:520]                             # second k-step tile, lane 0: row 0, k 32..39
    assert np.array_equal(tile1, codes[0, 32:40])


@pytest.mark.parametrize("dtype,K,N,layout", [(frt.BF16, 1024, 256, frt.W_PLAIN), (frt.BF16, 64, 64, frt.W_GATE_UP),
                                              (frt.E4M3, 256, 96, frt.W_PLAIN), (frt.E4M3, 128, 64, frt.W_GATE_UP)])
def test_weight_layout_is_a_bijection(dtype, K, N, layout):
    g = np.random.default_rng(K * N)
    codes = g.integers(0, 1 << (16 if dtype == frt.BF16 else 8), (K, N)).astype(np.uint16 if dtype == frt.BF16 else np.uint8)
    packed = frt.frt_weight_pack_host(codes, dtype, K, N, layout)
    assert packed.size == K * N * (2 if dtype == frt.BF16 else 1)
    assert np.array_equal(frt.frt_weight_unpack_host(packed, dtype, K, N, layout), codes)


@pytest.mark.parametrize("K,N,layout", [(128, 16, frt.W_PLAIN), (512, 96, frt.W_PLAIN), (256, 64, frt.W_GATE_UP)])
def test_mxfp4_weight_layout_is_a_bijection(K, N, layout):
    g = np.random.default_rng(K + N)
    codes = g.integers(0, 16, (K, N)).astype(np.uint8)
    scales = g.integers(0, 255, (K // 32, N)).astype(np.uint8)
    packed = frt.frt_weight_pack_mxfp4_host(codes, scales, K, N, layout)
    assert packed.size == frt.frt_weight_bytes(frt.MXFP4, K, N) == K * N // 2 + K * N // 32
    c2, s2 = frt.frt_weight_unpack_mxfp4_host(packed, K, N, layout)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)
    # every code nibble and every scale byte has its own place: an all-ones pattern fills
    # every byte of the packed weight
    full = frt.frt_weight_pack_mxfp4_host(np.full((K, N), 15, np.uint8), np.full((K // 32, N), 255, np.uint8),
                                          K, N, layout)
    assert np.all(full == 255)


def test_mxfp4_tile_structure():
    """Tile (column tile, k-step) = 1 KB of codes then 64 scale bytes; lane L = column L%16,
    MX block L/16 of the k-step: 32 consecutive k, two per byte, the even k in the low nibble."""
    K, N = 256, 32
    codes = ((np.arange(K)[:, None] + 3 * np.arange(N)[None, :]) % 16).astype(np.uint8)
    scales = (np.arange(K // 32)[:, None] * 40 + np.arange(N)[None, :]).astype(np.uint8)
    p = frt.frt_weight_pack_mxfp4_host(codes, scales, K, N, frt.W_PLAIN)
    tiles = p.reshape(-1, 1088)                      # (column tile, k-step) order, k-step fastest
    assert tiles.shape[0] == (N // 16) * (K // 128)
    t = tiles[1]                                     # column tile 0, k-step 1 (k 128..255)
    lane = 16 * 2 + 5                                # column 5, block 2 of the k-step: k 192..223
    slot = t[lane * 16:lane * 16 + 16]
    assert np.array_equal(slot & 15, codes[192:224:2, 5]) and np.array_equal(slot >> 4, codes[193:224:2, 5])
    assert t[1024 + lane] == scales[6, 5]            # block 6 of the column = k 192..223
    assert tiles[2][1024 + 3] == scales[0, 19]       # column tile 1, k-step 0, lane 3: column 19


def test_mxfp4_rejected_where_only_operand_formats_belong():
    assert frt.frt_operand_bytes(frt.MXFP4, 10, 1024) == 0
    assert frt.frt_weight_bytes(frt.MXFP4, 96, 64) == 0          # K must be a multiple of 128
    with pytest.raises(frt.FrtError):
        frt.frt_weight_pack_host(np.zeros((128, 16), np.uint8), frt.MXFP4, 128, 16)
    assert frt.frt_splitk_choose(50, 16384, 2048, frt.MXFP4) == frt.frt_splitk_choose(50, 16384, 2048, frt.E4M3)


def test_gate_up_layout_pairs_column_tiles():
    K, N = 32, 64
    codes = np.tile(np.arange(N, dtype=np.uint16), (K, 1))
    p = frt.frt_weight_pack_host(codes, frt.BF16, K, N, frt.W_GATE_UP).view(np.uint16)
    tiles = p.reshape(-1, 512)                       # one 1 KB tile per (column tile, k-step)
    assert tiles[0][0] == 0 and tiles[1][0] == N // 2      # gate tile 0, then up tile 0
    assert tiles[2][0] == 16 and tiles[3][0] == N // 2 + 16


def _st(name, *args):
    return getattr(frt.lib(), name)(*args)


@no_gpu
def test_producer_validation():
    f = "frt_residual_norm_quant"
    base = [None, 10, 1024, None, 1, 1.0, None, FAKE, FAKE, None, None, None, 1e-6, frt.BF16, 1.0, FAKE + 1 << 20]
    def call(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return _st(f, *a)
    assert call(a7=None) == frt.E_NULL                     # residual
    assert call(a8=None, a15=None) == frt.E_NULL           # neither output
    assert call(a1=0) == frt.E_SHAPE and call(a1=65) == frt.E_SHAPE
    assert call(a2=1000) == frt.E_SHAPE and call(a2=8192) == frt.E_SHAPE
    assert call(a13=7) == frt.E_DTYPE
    assert call(a13=frt.E4M3, a2=1056) == frt.E_SHAPE      # e4m3 needs K % 128
    assert call(a13=frt.E4M3, a14=0.0) == frt.E_ARG
    assert call(a3=FAKE, a4=0) == frt.E_SPLITK and call(a3=FAKE, a4=17) == frt.E_SPLITK
    assert call(a12=-1.0) == frt.E_ARG
    assert call(a7=FAKE + 4) == frt.E_ALIGN
    assert call(a15=FAKE + 64) == frt.E_ALIAS              # operand inside the residual


@no_gpu
def test_gemm_validation():
    f = "frt_skinny_gemm_splitk"
    A, W, P, O = FAKE, FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30)
    base = [None, 10, 1024, 1024, 4, frt.BF16, frt.W_PLAIN, A, W, None, 1.0, P, 4 * 10 * 1024 * 4,
            frt.EPI_NONE, None, frt.BF16, 1.0]
    def call(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return _st(f, *a)
    assert call(a7=None) == frt.E_NULL
    assert call(a5=9) == frt.E_DTYPE
    assert call(a1=0) == frt.E_SHAPE and call(a2=1000) == frt.E_SHAPE and call(a3=1000) == frt.E_SHAPE
    assert call(a4=3) == frt.E_SPLITK and call(a4=64) == frt.E_SPLITK
    assert call(a5=frt.E4M3, a4=16) == frt.E_SPLITK          # 8 k-steps cannot split 16 ways
    assert call(a12=100) == frt.E_WORKSPACE
    assert call(a11=None) == frt.E_NULL
    assert call(a13=9) == frt.E_ARG
    assert call(a13=frt.EPI_SILU_GATE_QUANT, a4=1, a14=O) == frt.E_ARG    # needs gate|up layout
    assert call(a13=frt.EPI_STORE_F32, a14=None) == frt.E_NULL
    assert call(a6=frt.W_GATE_UP, a2=1040) == frt.E_SHAPE
    assert call(a10=0.0) == frt.E_ARG
    assert call(a8=W + 8) == frt.E_ALIGN
    assert call(a11=A) == frt.E_ALIAS                         # partials over the operand


@no_gpu
def test_attention_and_pack_validation():
    f = "frt_attention_prefix"
    ws = frt.frt_attention_workspace_bytes(50, 8, 128, 850)
    assert ws > 0 and frt.frt_attention_workspace_bytes(50, 8, 64, 850) == 0
    base = [None, 50, 8, 128, 850, FAKE, FAKE + (1 << 30), FAKE + (2 << 30), 864, frt.BF16, 1.0,
            FAKE + (3 << 30), FAKE + (4 << 30), ws]
    def call(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return _st(f, *a)
    assert call(a5=None) == frt.E_NULL and call(a12=None) == frt.E_NULL
    assert call(a3=64) == frt.E_SHAPE and call(a2=0) == frt.E_SHAPE and call(a4=9000) == frt.E_SHAPE
    assert call(a4=49) == frt.E_SHAPE                        # kv_len must cover the M own rows
    assert call(a8=850) == frt.E_SHAPE and call(a8=832) == frt.E_SHAPE   # ldv: multiple of 32 >= kv_len
    assert call(a9=5) == frt.E_DTYPE
    assert call(a9=frt.E4M3, a10=-1.0) == frt.E_ARG
    if ws > 16:
        assert call(a13=ws - 1) == frt.E_WORKSPACE
    assert call(a11=FAKE) == frt.E_ALIAS
    assert call(a6=FAKE + 8) == frt.E_ALIGN
    qf = "frt_skinny_gemm_qkv"
    qbase = [None, 50, 1024, 8, 128, 1, frt.BF16, FAKE, FAKE + (1 << 30), None, 1.0, None, 0,
             FAKE + (2 << 30), FAKE + (3 << 30), FAKE + (4 << 30), 864]
    def qcall(**kw):
        a = list(qbase)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return _st(qf, *a)
    assert qcall(a13=None) == frt.E_NULL
    assert qcall(a4=100) == frt.E_SHAPE
    assert qcall(a5=4) == frt.E_NULL                         # split needs partials
    assert qcall(a5=4, a11=FAKE + (5 << 30), a12=10) == frt.E_WORKSPACE
    assert qcall(a14=FAKE + (2 << 30) + 64) == frt.E_ALIAS    # K rows overlap the Q rows
    assert qcall(a16=10) == frt.E_SHAPE                        # V^T rows shorter than M
    g = "frt_pack_weight"
    assert _st(g, None, 1024, 1024, None, None, frt.BF16, 0, FAKE, None) == frt.E_NULL
    assert _st(g, None, 1000, 1024, FAKE, None, frt.BF16, 0, FAKE + (1 << 30), None) == frt.E_SHAPE
    assert _st(g, None, 1024, 1024, FAKE, None, frt.E4M3, 0, FAKE + (1 << 30), None) == frt.E_NULL
    assert _st(g, None, 1024, 1024, FAKE, None, frt.BF16, 3, FAKE + (1 << 30), None) == frt.E_ARG
    assert _st(g, None, 1024, 1024, FAKE, None, frt.BF16, 0, FAKE + 1024, None) == frt.E_ALIAS
    r = "frt_splitk_reduce"
    assert _st(r, None, 10, 1024, 4, None, 1.0, None, frt.EPI_STORE_F32, FAKE, frt.F32, 1.0) == frt.E_NULL
    assert _st(r, None, 10, 1024, 4, FAKE, 1.0, None, frt.EPI_NONE, FAKE + (1 << 30), frt.F32, 1.0) == frt.E_ARG


@no_gpu
def test_chain_validation():
    ptrs = [FAKE + i * (1 << 28) for i in range(2)]
    d, keep = frt.make_chain_desc(2, 2, 50, 1024, 8, 128, 800, 4096, frt.BF16, 1e-6, (0, 0, 0, 0),
                                  ptrs, ptrs, ptrs, ptrs)
    n = frt.frt_layer_chain_arena_bytes(d)
    assert n > 2 * 50 * 1024 * 4
    h = ctypes.c_void_p()
    lib = frt.lib()
    assert lib.frt_layer_chain_create(ctypes.byref(d), None, n, None, ctypes.byref(h)) == frt.E_NULL
    assert lib.frt_layer_chain_create(ctypes.byref(d), FAKE, n - 1, None, ctypes.byref(h)) == frt.E_WORKSPACE
    d.head_dim = 64
    assert frt.frt_layer_chain_arena_bytes(d) == 0
    assert lib.frt_layer_chain_create(ctypes.byref(d), FAKE, n, None, ctypes.byref(h)) == frt.E_SHAPE
    d.head_dim = 128
    d.dtype = frt.E4M3
    assert lib.frt_layer_chain_create(ctypes.byref(d), FAKE, n, None, ctypes.byref(h)) == frt.E_NULL  # no scales
    d.dtype = frt.BF16
    d.splits_up = 3
    assert lib.frt_layer_chain_create(ctypes.byref(d), FAKE, n, None, ctypes.byref(h)) == frt.E_SPLITK
    assert lib.frt_layer_chain_buffer(None, b"x_in", None, None) == frt.E_STATE
    assert lib.frt_layer_chain_run(None, None) == frt.E_STATE
    assert lib.frt_layer_chain_calibrate(None, None, None) == frt.E_STATE
    assert lib.frt_layer_chain_destroy(None) == frt.E_STATE
    assert lib.frt_layer_chain_kernel_count(None) == -1
    assert lib.frt_layer_chain_state_bytes(None) == 0
    assert lib.frt_layer_chain_snapshot(None, None, FAKE, 1 << 20) == frt.E_STATE
    assert lib.frt_layer_chain_restore(None, None, FAKE, 1 << 20) == frt.E_STATE
    # keep_intermediates grows the arena by the per-(step, layer) debug buffers
    d.splits_up = 0
    d.keep_intermediates = 1
    assert frt.frt_layer_chain_arena_bytes(d) > n
