"""Comparison helpers for the parity tests (test-side arithmetic only).

Tie band: the oracle rounds float64 values, the GPU rounds float32 values computed in
another order, so a code may legitimately differ where the exact value sits within the
GPU's float32 error of a rounding boundary.  A GPU code is accepted when it is a correct
rounding of some value within TAU * mag of the oracle's exact pre-rounding value v, i.e.
when it lies (in value order) between encode(v - TAU*mag) and encode(v + TAU*mag); mag is
the size of the summands that produced v, so cancellation cannot shrink the band below
float32's own error.  TAU = 2**-17 is 128 float32 ulps of the summands.  Rounding is
monotone, so the interval test is exact.

Count limit: at most max_frac of the codes may differ, which catches a drift that stays
inside the band.  A differing code whose oracle value sits within FP32_TIE (relative to
the value itself) of the midpoint between the two codes is a tie that float32 cannot
decide the way float64 does (its own rounding of the scale alone is 2**-24); such codes
are not counted.  They are common only where the inputs are themselves coarse, e.g. a
single key, whose attention output is a bf16 value of V, over a scale that is a bf16
maximum / 448.
"""
import numpy as np

from oracle import codec

TAU = 2.0 ** -17
FP32_TIE = 2.0 ** -21


def _ordinal(codes, dtype):
    c = np.asarray(codes).astype(np.int64)
    if dtype == "bf16":
        mag, sign = c & 0x7FFF, (c >> 15) & 1
    else:
        mag, sign = c & 0x7F, (c >> 7) & 1
    return np.where(sign == 1, -mag, mag)


def check_codes(gpu_codes, v, mag, dtype, tau=TAU, max_frac=0.01, label=""):
    """Assert GPU codes equal the oracle's up to the tie band; return (n_diff, n_total)."""
    gpu_codes = np.asarray(gpu_codes)
    v = np.asarray(v, dtype=np.float64)
    mag = np.broadcast_to(np.asarray(mag, dtype=np.float64), v.shape)
    want = codec.encode(v, dtype)
    assert gpu_codes.shape == want.shape, (gpu_codes.shape, want.shape)
    diff = np.flatnonzero(gpu_codes.ravel() != want.ravel())
    n_ties = 0
    if len(diff):
        vv = v.ravel()[diff]
        band = tau * mag.ravel()[diff]
        lo = _ordinal(codec.encode(vv - band, dtype), dtype)
        hi = _ordinal(codec.encode(vv + band, dtype), dtype)
        g = _ordinal(gpu_codes.ravel()[diff], dtype)
        ok = (g >= lo) & (g <= hi)
        bad = diff[~ok]
        if len(bad):
            i = bad[0]
            raise AssertionError(
                f"{label}: {len(bad)} codes outside the tie band of {len(diff)} differing "
                f"(of {v.size}); first at flat index {i}: gpu {int(gpu_codes.ravel()[i]):#x} "
                f"oracle {int(want.ravel()[i]):#x} value {v.ravel()[i]!r} mag {mag.ravel()[i]!r}")
        w = want.ravel()[diff]
        mid = 0.5 * (codec.decode(gpu_codes.ravel()[diff], dtype) + codec.decode(w, dtype))
        adjacent = np.abs(g - _ordinal(w, dtype)) == 1
        n_ties = int(np.count_nonzero(adjacent & (np.abs(vv - mid) <= FP32_TIE * np.abs(vv))))
    assert len(diff) - n_ties <= max_frac * v.size, (
        f"{label}: {len(diff)} of {v.size} codes differ ({n_ties} of them at a float32 tie)")
    return len(diff), v.size


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b.ravel())
    return float(np.linalg.norm((a - b).ravel()) / (den if den > 0 else 1.0))


def bf16_values(bits):
    return codec.bf16_decode(np.asarray(bits).view(np.uint16))


def silu_gate_mag(c, a_dec, w_dec, act, s_w, dtype, out_scale):
    """Summand sizes of z = SiLU(gate) * up for the tie band: the GEMM sums feeding gate
    and up (|SiLU'| <= 1.1) and the product itself, scaled like the rounded value."""
    from oracle import ref
    g_mag = (np.abs(a_dec) @ np.abs(w_dec)) * act * (np.asarray(s_w)[None, :] if s_w is not None else 1.0)
    n2 = c.shape[1] // 2
    gte, up = c[:, :n2], c[:, n2:]
    mag = 1.1 * np.abs(up) * g_mag[:, :n2] + np.abs(ref.silu(gte)) * g_mag[:, n2:] + np.abs(ref.silu(gte) * up)
    return mag / out_scale if dtype == "e4m3" else mag


class Canaries:
    """Device buffers with PAD canary bytes on each side (canary-guarded outputs):
    `bytes` / `f32` hand out the inner region, `check` asserts that no kernel wrote past
    either end of any buffer handed out."""
    PAD = 256
    BYTE = 0x5A

    def __init__(self):
        self.bufs = []

    def bytes(self, nbytes):
        import torch
        n = max(int(nbytes), 16)
        buf = torch.full((n + 2 * self.PAD,), self.BYTE, dtype=torch.uint8, device="cuda")
        self.bufs.append((buf, n))
        return buf[self.PAD:self.PAD + n]

    def f32(self, *shape):
        import torch
        n = int(np.prod(shape)) * 4
        buf = torch.full((n + 2 * self.PAD,), self.BYTE, dtype=torch.uint8, device="cuda")
        self.bufs.append((buf, n))
        return buf[self.PAD:self.PAD + n].view(torch.float32).view(*shape)

    def check(self):
        import torch
        torch.cuda.synchronize()
        for i, (buf, n) in enumerate(self.bufs):
            head = buf[:self.PAD].cpu().numpy()
            tail = buf[self.PAD + n:].cpu().numpy()
            assert np.all(head == self.BYTE), f"buffer {i} ({n} bytes): canary before it overwritten"
            assert np.all(tail == self.BYTE), f"buffer {i} ({n} bytes): canary after it overwritten"
        return len(self.bufs)


# Parity figures measured during the session, printed in pytest's terminal summary (so a
# quiet run still reports them): label -> text.
FIGURES = {}


def record(label, text):
    FIGURES[label] = text


def e4m3_products_exact(M):
    """The library multiplies e4m3 weights by e4m3 activations with exact products (codes
    decoded to bf16, fp32 sums) when the GEMM has at most 16 rows, and with the fp8 MFMA,
    whose internal sum keeps about 13 bits (~1.5e-5 relative on partial sums), above."""
    return M <= 16


def partial_bar(wdtype, M):
    """Relative L2 bar of fp32 partial sums against the float64 products: 1e-5 for exact
    products (bf16 weights; e4m3 weights at M <= 16), 1e-4 through the fp8 and FP4 x FP8
    MFMAs' internal sums."""
    if wdtype == "bf16" or (wdtype == "e4m3" and e4m3_products_exact(M)):
        return 1e-5
    return 1e-4
