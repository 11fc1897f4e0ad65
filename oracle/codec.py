"""Software number formats for the oracle: float64 <-> bfloat16, OCP E4M3FN and OCP MXFP4 codes.

TEST INFRASTRUCTURE ONLY.  Nothing outside ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU
library never calls into it and it never calls into the GPU library.

Why the formats matter: the pages' static-quantisation section
("静态量化改变了两次矩阵乘之间的工作" in the observation-age notes
"思考探索：具身推理加速，先看动作执行时观测有多旧") has the producer of a GEMM
input write it directly in the low-precision format the GEMM consumes (FP8,
with a scale fixed in advance), and the FlashRT-PAI news summary
("它优化的是“接力方式”") names FP8 as the precision of the fused
action-decoder layer.  The pages fix neither the FP8 flavour nor the rounding;
the reading taken here is OCP E4M3FN (bias 7, largest finite 448, no
infinities, one NaN mantissa pattern), round to nearest with ties to even,
saturating at +-448, signed zero kept.  bfloat16 is IEEE-style binary16 with
an 8-bit exponent (bias 127) and 7 fraction bits, round to nearest even.

Both encoders work from the definition of the format (exponent, quantum,
round-to-nearest-even of the scaled magnitude in float64), not from bit
tricks on a narrower float, so they are independent of how any GPU rounds.
"""
import numpy as np

E4M3_MAX = 448.0          # 1.75 * 2**8: exponent field 15, mantissa 6
E4M3_NAN = 0x7F


def _as_f64(v):
    return np.asarray(v, dtype=np.float64)


def _floor_log2(a):
    """floor(log2(a)) for finite a > 0, exact (frexp returns a = f * 2**e, f in [0.5, 1))."""
    _, e = np.frexp(a)
    return e.astype(np.int64) - 1


# ---------------------------------------------------------------- bfloat16

def bf16_encode(v):
    """float64 array -> bfloat16 bit patterns (uint16), round to nearest, ties to even.

    Normal range: a = |v| in [2**-126, 2**128); quantum 2**(E-7) with E = floor(log2 a);
    the 8-bit significand m = rne(a / quantum) lies in [128, 256]; m == 256 carries into
    the exponent.  Below 2**-126 the quantum is fixed at 2**-133 (subnormals).  Values
    that round past the largest finite number become infinity; NaN becomes 0x7FC0.
    """
    v = _as_f64(v)
    sign = np.signbit(v).astype(np.uint32) << 15
    a = np.abs(v)
    out = np.zeros(a.shape, np.uint32)

    nan = np.isnan(a)
    inf = np.isinf(a)
    fin = ~(nan | inf)
    sub = fin & (a < 2.0 ** -126)
    nrm = fin & ~sub

    # subnormal: m in [0, 128]; m == 128 is exactly the smallest normal (code 0x0080)
    m_sub = np.rint(np.ldexp(a[sub], 133))
    out[sub] = m_sub.astype(np.uint32)

    an = a[nrm]
    e = _floor_log2(an)
    m = np.rint(np.ldexp(an, (7 - e)))          # exact scaling by a power of two, then RNE
    carry = m == 256.0
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 128.0, m)
    code = ((e + 127).astype(np.int64) << 7) | (m.astype(np.int64) - 128)
    code = np.where(e > 127, 0x7F80, code)        # rounded past the largest finite value
    out[nrm] = code.astype(np.uint32)

    out[inf] = 0x7F80
    out = out | sign
    out[nan] = 0x7FC0
    return out.astype(np.uint16)


def bf16_decode(c):
    """bfloat16 bit patterns -> float64 values."""
    c = np.asarray(c).astype(np.int64)
    s = np.where((c >> 15) & 1, -1.0, 1.0)
    e = (c >> 7) & 0xFF
    m = (c & 0x7F).astype(np.float64)
    val = np.where(e == 0, np.ldexp(m, -133), np.ldexp(1.0 + m / 128.0, e - 127))
    val = np.where(e == 255, np.where(m == 0, np.inf, np.nan), val)
    return s * val


def bf16_round(v):
    """Round float64 values to the nearest bfloat16 value (ties to even)."""
    return bf16_decode(bf16_encode(v))


# ---------------------------------------------------------------- OCP E4M3FN

def e4m3_encode(v):
    """float64 array -> OCP E4M3FN codes (uint8): RNE, saturating to +-448, -0 kept, NaN -> 0x7F.

    Normal range: a in [2**-6, 448]; E = floor(log2 a) in [-6, 8], quantum 2**(E-3), the
    4-bit significand q = rne(a / quantum) in [8, 16], q == 16 carries.  Below 2**-6 the
    quantum is 2**-9 (subnormals, q in [0, 8]; q == 8 is exactly the smallest normal).
    """
    v = _as_f64(v)
    sign = np.signbit(v).astype(np.uint32) << 7
    a = np.abs(v)
    out = np.zeros(a.shape, np.uint32)

    nan = np.isnan(a)
    sat = ~nan & (a >= E4M3_MAX)                  # includes +-inf
    sub = ~nan & (a < 2.0 ** -6)
    nrm = ~(nan | sat | sub)

    out[sub] = np.rint(np.ldexp(a[sub], 9)).astype(np.uint32)

    an = a[nrm]
    e = _floor_log2(an)
    q = np.rint(np.ldexp(an, 3 - e))
    carry = q == 16.0
    e = np.where(carry, e + 1, e)
    q = np.where(carry, 8.0, q)
    out[nrm] = (((e + 7) << 3) | (q.astype(np.int64) - 8)).astype(np.uint32)

    out[sat] = 0x7E
    out = out | sign
    out[nan] = E4M3_NAN
    return out.astype(np.uint8)


def e4m3_decode(c):
    """OCP E4M3FN codes -> float64 values (0x7F / 0xFF decode to NaN)."""
    c = np.asarray(c).astype(np.int64)
    s = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    val = np.where(e == 0, np.ldexp(m, -9), np.ldexp(1.0 + m / 8.0, e - 7))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return s * val


def e4m3_round(v):
    """Round float64 values to the nearest E4M3FN value (saturating)."""
    return e4m3_decode(e4m3_encode(v))


# ---------------------------------------------------------------- OCP MXFP4 (E2M1 elements, E8M0 block scales)
#
# The pages run the fused action decoder's weights at 4 bits on their NVIDIA target
# (the FlashRT-PAI abstract and news summary).  On gfx950 the matrix cores take OCP
# microscaling formats natively, so the 4-bit weights here are OCP MXFP4 ("OCP
# Microscaling Formats (MX) Specification" v1.0): blocks of 32 consecutive elements along
# K share one E8M0 scale X = 2**e (e in [-127, 127], byte e + 127); each element is FP4
# E2M1 (sign, 2 exponent bits with bias 1, 1 mantissa bit; magnitudes 0, 0.5, 1, 1.5,
# 2, 3, 4, 6; no infinities or NaN).  The block exponent is floor(log2(max |v|)) minus the
# largest element exponent (2), so max |v| / X lies in [4, 8); elements are v / X rounded
# to nearest, ties to even, saturating at +-6.

FP4_MAX = 6.0
MX_BLOCK = 32


def fp4_encode(v):
    """float64 array -> FP4 E2M1 codes (uint8, low 4 bits): RNE, saturating to +-6, -0 kept.

    Below 1 the quantum is 0.5 (exponent field 0: q in [0, 2], q == 2 is exactly 1.0);
    from 1 up, E = floor(log2 a) in [0, 2], quantum 2**(E-1), q = rne(a / quantum) in
    [2, 4] and q == 4 carries into the exponent; past the largest exponent the code
    saturates at 6.
    """
    v = _as_f64(v)
    sign = np.signbit(v).astype(np.uint32) << 3
    a = np.abs(v)
    out = np.zeros(a.shape, np.uint32)
    sub = a < 1.0
    out[sub] = np.rint(a[sub] * 2.0).astype(np.uint32)          # 0, 1 (0.5) or 2 (1.0)
    nrm = ~sub & (a < 8.0)
    an = a[nrm]
    e = _floor_log2(an)
    q = np.rint(np.ldexp(an, 1 - e))
    carry = q == 4.0
    e = np.where(carry, e + 1, e)
    q = np.where(carry, 2.0, q)
    code = ((e + 1) << 1) | (q.astype(np.int64) - 2)
    out[nrm] = np.minimum(code, 7).astype(np.uint32)             # exponent past 2 -> 6
    out[~sub & ~nrm] = 7                                        # |v| >= 8 (and inf): 6
    return (out | sign).astype(np.uint8)


def fp4_decode(c):
    """FP4 E2M1 codes -> float64 values."""
    c = np.asarray(c).astype(np.int64)
    s = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    return s * np.where(e == 0, m * 0.5, np.ldexp(1.0 + m / 2.0, e - 1))


def mxfp4_encode(w):
    """MXFP4 along axis 0 (K) of w [K][N] (K a multiple of 32).

    Returns (codes [K][N] uint8 FP4, scale bytes [K/32][N] uint8 E8M0, X [K/32][N] float64).
    A block whose largest magnitude is 0 gets scale byte 0 and zero codes.
    """
    w = _as_f64(w)
    K, N = w.shape
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    blocks = w.reshape(K // MX_BLOCK, MX_BLOCK, N)
    amax = np.max(np.abs(blocks), axis=1)                        # [K/32][N]
    nz = amax > 0
    e = np.where(nz, _floor_log2(np.where(nz, amax, 1.0)) - 2, -127)
    e = np.clip(e, -127, 127)
    X = np.ldexp(1.0, e)
    codes = fp4_encode(blocks / X[:, None, :]).reshape(K, N)     # exact scaling by 2**-e
    return codes, (e + 127).astype(np.uint8), X


def mxfp4_decode(codes, scale_bytes):
    """MXFP4 codes [K][N] with E8M0 scale bytes [K/32][N] -> float64 values [K][N]."""
    K, N = codes.shape
    X = np.ldexp(1.0, np.asarray(scale_bytes).astype(np.int64) - 127)
    return (fp4_decode(codes).reshape(K // MX_BLOCK, MX_BLOCK, N) * X[:, None, :]).reshape(K, N)


# ---------------------------------------------------------------- generic

def encode(v, dtype):
    if dtype == "bf16":
        return bf16_encode(v)
    if dtype == "e4m3":
        return e4m3_encode(v)
    raise ValueError(dtype)


def decode(c, dtype):
    if dtype == "bf16":
        return bf16_decode(c)
    if dtype == "e4m3":
        return e4m3_decode(c)
    raise ValueError(dtype)

