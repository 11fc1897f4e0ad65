"""The GPU's float32 -> bf16 and float32 -> e4m3 conversions against the oracle's codecs,
bit for bit (MI355X only).

The producer kernel is made to quantise chosen float32 values exactly: with a constant
negative residual row, ada_scale = -1 and ada_shift = v, its output before rounding is
xhat * (1 + (-1)) + v = -0 + v = v for every v (including -0, infinities and NaN), and an
e4m3 activation scale of 1 divides exactly.  The codes it writes are then the hardware
path's rounding of v (gfx950's pack-converts, behind the kernel's saturating clamp for
e4m3), and must equal codec.bf16_encode(v) / codec.e4m3_encode(v) exactly:
  - every finite value of each format, every rounding midpoint between neighbours, and
    those points moved by 1..4 float32 ulps either way (ties to even, and no double
    rounding near a tie);
  - the subnormal ranges and their boundaries (the smallest subnormals, half of them,
    the subnormal/normal boundary);
  - e4m3 saturation: 448, the 448/480 midpoint 464 and its neighbours, larger values,
    infinities (all saturate to +-448 by the clamp);
  - NaN (e4m3: 0x7F; bf16: any NaN code -- the format leaves the payload open);
  - about 10^7 random float32 values: random bit patterns, and log-uniform magnitudes
    over each format's range.
The same device conversions serve every kernel that writes a bf16 or e4m3 value (the
producers, the GEMM epilogues, attention's operand), through the shared helpers.

Pages: observation-age notes "思考探索：具身推理加速，先看动作执行时观测有多旧", section
"CUDA Graph 与图化简分别省掉什么" (at low precision the rounding and its error must be
checked, not assumed); section "静态量化改变了两次矩阵乘之间的工作" (FP8 conversion at
every GEMM input).
"""
import numpy as np
import pytest
import torch

from oracle import codec
from tests.helpers import record

pytestmark = pytest.mark.gpu

K = 4096          # values per producer call (one row)
BATCH = 256       # calls per device round trip


@pytest.fixture(scope="module")
def F():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X GPU")
    from gemm_chains_amd import device, frt
    frt.lib()
    return frt, device


def _f32(bits):
    return np.asarray(bits, np.uint32).view(np.float32)


def _near(bits_center, spread=4):
    """bit patterns within +-spread ulps of each centre (same sign; no wrap into NaN/inf)."""
    c = np.asarray(bits_center, np.int64)
    out = [c + d for d in range(-spread, spread + 1)]
    out = np.concatenate(out)
    mag = out & 0x7FFFFFFF
    return out[(out >= 0) & (out <= 0xFFFFFFFF) & (mag <= 0x7F800000)].astype(np.uint32)


def _bf16_points():
    codes = np.arange(0, 0x7F80, dtype=np.uint32)                 # finite non-negative bf16
    exact = codes << 16
    mids = exact[:-1] + 0x8000                                    # midpoint to the next code
    pts = np.concatenate([_near(exact), _near(mids), _near(np.array([0x7F7F8000, 0x7F800000]))])
    pts = np.concatenate([pts, pts | 0x80000000])
    return np.unique(pts)


def _e4m3_points():
    vals = codec.e4m3_decode(np.arange(0, 0x7F))                  # finite non-negative e4m3
    vals = np.unique(vals)
    mids = (vals[:-1] + vals[1:]) / 2
    extra = np.array([448.0, 464.0, 480.0, 500.0, 1e4, 3e38, 2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11,
                      2.0 ** -7 - 2.0 ** -11, 2.0 ** -6 - 2.0 ** -10, 2.0 ** -6, 2.0 ** -20, 1e-30, 1e-40])
    centres = np.concatenate([vals, mids, extra]).astype(np.float32).view(np.uint32)
    pts = np.concatenate([_near(centres), np.array([0x7F800000], np.uint32)])
    pts = np.concatenate([pts, pts | 0x80000000])
    return np.unique(pts)


def _random_points(seed, n, lo_exp, hi_exp):
    g = np.random.default_rng(seed)
    raw = g.integers(0, 2 ** 32, size=n // 2, dtype=np.uint64).astype(np.uint32)
    raw = raw[(raw & 0x7F800000) != 0x7F800000]                   # NaN/inf handled separately
    mag = np.exp2(g.uniform(lo_exp, hi_exp, size=n - n // 2))
    sgn = np.where(g.integers(0, 2, size=mag.size) == 1, -1.0, 1.0)
    return np.concatenate([raw, (sgn * mag).astype(np.float32).view(np.uint32)])


def _convert(frt, device, bits, dtype):
    """Quantise the float32 values `bits` (uint32 patterns) with the producer kernel, K per
    call; return the codes (uint16 bf16 / uint8 e4m3), one per value."""
    n = bits.size
    calls = (n + K - 1) // K
    vals = np.zeros(calls * K, np.float32)
    vals[:n] = _f32(bits)
    res = torch.full((K,), -0.75, dtype=torch.float32, device="cuda")      # constant negative row
    ada = torch.full((K,), -1.0, dtype=torch.float32, device="cuda")
    ob = frt.frt_operand_bytes(dtype, 1, K)
    out = []
    for b0 in range(0, calls, BATCH):
        nb = min(BATCH, calls - b0)
        shifts = device.to_dev(vals[b0 * K:(b0 + nb) * K].reshape(nb, K))
        ops = torch.empty((nb, ob), dtype=torch.uint8, device="cuda")
        for i in range(nb):
            frt.frt_residual_norm_quant(1, K, None, 1, 1.0, None, res, None, None, ada, shifts[i], 1e-6, dtype,
                                        1.0, ops[i])
        host = ops.cpu().numpy()
        for i in range(nb):
            out.append(frt.frt_operand_unpack_host(host[i], dtype, 16, K)[0])
    return np.concatenate(out)[:n]


def _compare(got, bits, dtype):
    v = _f32(bits).astype(np.float64)
    want = codec.encode(v, dtype)
    nan = np.isnan(v)
    if dtype == "bf16":
        g = got.astype(np.uint32)
        assert np.all(((g & 0x7F80) == 0x7F80) & ((g & 0x7F) != 0) | ~nan), "bf16 NaN must stay NaN"
    skip = nan if dtype == "bf16" else np.zeros_like(nan)
    bad = np.flatnonzero((got != want) & ~skip)
    if bad.size:
        i = bad[0]
        raise AssertionError(f"{dtype}: {bad.size} of {bits.size} codes differ; first: value {v[i]!r} "
                             f"(bits {int(bits[i]):#010x}) gpu {int(got[i]):#x} oracle {int(want[i]):#x}")


@pytest.mark.parametrize("dtype", ["bf16", "e4m3"])
def test_converter_edges(F, dtype):
    frt, device = F
    bits = _bf16_points() if dtype == "bf16" else _e4m3_points()
    bits = np.concatenate([bits, np.array([0x7FC00000, 0xFFC00000, 0x7F800001, 0x7FBFFFFF], np.uint32)])
    got = _convert(frt, device, bits, frt.DTYPES[dtype])
    _compare(got, bits, dtype)
    print(f"{dtype} converter: {bits.size} edge values bit-exact", flush=True)
    record(f"converter {dtype} edges", f"{bits.size} values bit-exact")


@pytest.mark.parametrize("dtype", ["bf16", "e4m3"])
def test_converter_random(F, dtype):
    frt, device = F
    lo, hi = (-140, 128) if dtype == "bf16" else (-12, 9.5)
    bits = _random_points(17 if dtype == "bf16" else 18, 10_000_000, lo, hi)
    got = _convert(frt, device, bits, frt.DTYPES[dtype])
    _compare(got, bits, dtype)
    print(f"{dtype} converter: {bits.size} random values bit-exact", flush=True)
    record(f"converter {dtype} random", f"{bits.size} values bit-exact")
