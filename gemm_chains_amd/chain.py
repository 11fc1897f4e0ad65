"""Plumbing around the chain entry points: pack a layer stack, own the arena, fill and
read named buffers.  All arithmetic runs in the library's kernels."""
import numpy as np
import torch

from . import device, frt

BUFFER_DTYPES = {"x_in": np.float32, "x_out": np.float32, "mod": np.float32, "act_scale": np.float32,
                 "k_cache": np.int16, "v_cache": np.int16, "h": np.float32,
                 "dbg_h_attn": np.float32, "dbg_h_mlp": np.float32,
                 "dbg_p_o": np.float32, "dbg_p_down": np.float32, "dbg_q": np.int16,
                 "dbg_k_own": np.int16, "dbg_v_own": np.int16,
                 "dbg_a_qkv": np.uint8, "dbg_a_o": np.uint8, "dbg_a_up": np.uint8, "dbg_a_down": np.uint8}
_TORCH = {np.float32: torch.float32, np.int16: torch.int16, np.uint8: torch.uint8}


class PackedLayers:
    """GPU-packed weights of a layer stack (bf16 master weights in, bf16 or e4m3 out)."""

    def __init__(self, layers, dims, dtype, stream=None):
        self.dtype = dtype
        self.w = {k: [] for k in ("qkv", "o", "up", "down")}
        self.s = {k: [] for k in ("qkv", "o", "up", "down")}
        for lw in layers:
            for name, layout in (("qkv", frt.W_PLAIN), ("o", frt.W_PLAIN), ("up", frt.W_GATE_UP),
                                 ("down", frt.W_PLAIN)):
                pk, cs = device.pack_weight(lw[name], dtype, layout, stream=stream)
                self.w[name].append(pk)
                self.s[name].append(cs)

    def nbytes(self):
        return sum(t.numel() for v in self.w.values() for t in v)


class Chain:
    """One chain handle with its own arena (a torch uint8 CUDA tensor)."""

    def __init__(self, dims, packed, splits=(0, 0, 0, 0), use_graph=True, keep_intermediates=False, eps=1e-6,
                 stream=None, prefetch_next=False):
        e4 = packed.dtype == frt.E4M3
        self.dims = dims
        self.desc, self._keep = frt.make_chain_desc(
            dims["layers"], dims["steps"], dims["M"], dims["hidden"], dims["n_heads"], dims["head_dim"],
            dims["prefix"], dims["mlp"], packed.dtype, eps, splits,
            packed.w["qkv"], packed.w["o"], packed.w["up"], packed.w["down"],
            packed.s["qkv"] if e4 else None, packed.s["o"] if e4 else None,
            packed.s["up"] if e4 else None, packed.s["down"] if e4 else None,
            use_graph=use_graph, keep_intermediates=keep_intermediates, prefetch_next=prefetch_next)
        self.packed = packed
        nbytes = frt.frt_layer_chain_arena_bytes(self.desc)
        if nbytes == 0:
            raise ValueError("invalid chain description")
        self.arena = torch.zeros(nbytes, dtype=torch.uint8, device=device.DEV)
        torch.cuda.synchronize()
        self.handle = frt.frt_layer_chain_create(self.desc, self.arena, nbytes, stream)

    def view(self, name):
        ptr, nbytes = frt.frt_layer_chain_buffer(self.handle, name)
        off = ptr - self.arena.data_ptr()
        dt = BUFFER_DTYPES[name]
        return self.arena[off:off + nbytes].view(_TORCH[dt])

    def write(self, name, array):
        v = self.view(name)
        src = torch.from_numpy(np.ascontiguousarray(array).view(BUFFER_DTYPES[name]).ravel())
        assert src.numel() == v.numel(), (name, src.numel(), v.numel())
        v.copy_(src.to(device.DEV))

    def read(self, name):
        return self.view(name).cpu().numpy()

    def run(self, stream=None):
        frt.frt_layer_chain_run(self.handle, stream)

    def calibrate(self, stream=None):
        """Static e4m3 activation scales [layers][4] from one recorded bf16 run (device tensor)."""
        out = torch.empty((self.dims["layers"], 4), dtype=torch.float32, device=device.DEV)
        frt.frt_layer_chain_calibrate(self.handle, out, stream)
        return out

    def kernel_count(self):
        return frt.frt_layer_chain_kernel_count(self.handle)

    def state_bytes(self):
        return frt.frt_layer_chain_state_bytes(self.handle)

    def snapshot(self, capsule=None, stream=None):
        """Copy the persistent state into a capsule (a uint8 CUDA tensor; new if None)."""
        n = self.state_bytes()
        if capsule is None:
            capsule = device.empty_bytes(n)
        frt.frt_layer_chain_snapshot(self.handle, capsule, capsule.numel(), stream)
        return capsule

    def restore(self, capsule, stream=None):
        """Copy a capsule back into this chain's persistent state (fixed addresses)."""
        frt.frt_layer_chain_restore(self.handle, capsule, capsule.numel(), stream)

    def close(self):
        if self.handle is not None:
            frt.frt_layer_chain_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def load_workload(chain, wl, act_scales=None):
    """Fill the named input buffers from a synthetic workload (synth.workload4)."""
    chain.write("x_in", wl["x0"])
    chain.write("mod", wl["mod"])
    d = wl["dims"]
    if d["prefix"]:
        # prefix keys at the head of each layer's key cache; prefix values transposed at the
        # head of each row of the value cache; the own rows are written by the chain
        P, hd, T = d["prefix"], d["head_dim"], d["prefix"] + d["M"]
        ldv = (T + 31) // 32 * 32
        kc = chain.view("k_cache").view(d["layers"], T, hd)
        vc = chain.view("v_cache").view(d["layers"], hd, ldv)
        for l, lw in enumerate(wl["layers"]):
            kc[l, :P].copy_(torch.from_numpy(np.ascontiguousarray(lw["k_prefix"]).view(np.int16)).to(device.DEV))
            vt = np.ascontiguousarray(np.asarray(lw["v_prefix"]).T).view(np.int16)
            vc[l, :, :P].copy_(torch.from_numpy(vt).to(device.DEV))
    L = d["layers"]
    chain.write("act_scale", np.ones((L, 4), np.float32) if act_scales is None
                else np.asarray(act_scales, np.float32).reshape(L, 4))
