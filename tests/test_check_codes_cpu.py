"""The code comparison used by every parity test (tests/helpers.py check_codes), on the
CPU: what it accepts and what it rejects, on values built to sit at rounding midpoints,
inside the tie band, and outside it."""
import numpy as np
import pytest

import synth
from oracle import codec, ref
from tests import chain_parity as cp
from tests.helpers import TAU, check_codes


def _midpoints(dtype, n, seed):
    """n values exactly halfway between two adjacent codes (positive and negative), and
    the two codes (below and above in magnitude)."""
    rng = np.random.default_rng(seed)
    if dtype == "e4m3":
        codes = np.arange(0x08, 0x7E, dtype=np.uint8)          # normals, below the maximum
        grid = codec.decode(codes, "e4m3")
    else:
        codes = np.arange(0x3C00, 0x4400, dtype=np.uint16)
        grid = codec.bf16_decode(codes)
    i = rng.integers(0, grid.size - 1, n)
    neg = rng.random(n) < 0.5
    sign_bit = 0x80 if dtype == "e4m3" else 0x8000
    lo = np.where(neg, codes[i] | sign_bit, codes[i]).astype(codes.dtype)
    hi = np.where(neg, codes[i + 1] | sign_bit, codes[i + 1]).astype(codes.dtype)
    return 0.5 * (grid[i] + grid[i + 1]) * np.where(neg, -1.0, 1.0), lo, hi


def _other(got, lo, hi):
    return np.where(got == lo, hi, lo)


@pytest.mark.parametrize("dtype", ["e4m3", "bf16"])
def test_flipped_midpoints_are_ties_and_not_counted(dtype):
    m, lo, hi = _midpoints(dtype, 400, 3)
    v = m * (1.0 + 2.0 ** -26)                             # a float32 rounding away from the tie
    got = codec.encode(v, dtype).copy()
    got[:120] = _other(got[:120], lo[:120], hi[:120])      # 30 % flipped, all at a tie
    n, tot = check_codes(got, v, np.abs(v), dtype)
    assert (n, tot) == (120, 400)


@pytest.mark.parametrize("dtype", ["e4m3", "bf16"])
def test_in_band_flips_off_the_midpoint_are_counted(dtype):
    # values a quarter of a code step from the midpoint: not ties, but inside a band
    # widened by a large summand size (mag), so only the count limit can catch them
    rng = np.random.default_rng(5)
    m, lo, hi = _midpoints(dtype, 400, 4)
    dec = codec.bf16_decode if dtype == "bf16" else (lambda c: codec.decode(c, "e4m3"))
    step = np.abs(dec(hi) - dec(lo))
    v = m + 0.25 * step * np.where(rng.random(400) < 0.5, -1.0, 1.0)
    mag = 2.0 * step / TAU
    want = codec.encode(v, dtype)
    got = want.copy()
    got[:8] = _other(want[:8], lo[:8], hi[:8])             # 2 %: inside the band, off the tie
    with pytest.raises(AssertionError, match="8 of 400 codes differ"):
        check_codes(got, v, mag, dtype)
    got[3:] = want[3:]                                      # 0.75 %: within the count limit
    assert check_codes(got, v, mag, dtype) == (3, 400)


@pytest.mark.parametrize("dtype", ["e4m3", "bf16"])
def test_flips_outside_the_band_are_rejected(dtype):
    m, lo, hi = _midpoints(dtype, 64, 6)
    v = m * 1.01                                           # well off any tie
    got = codec.encode(v, dtype).copy()
    got[0] = _other(got[:1], lo[:1], hi[:1])[0]
    if got[0] == codec.encode(v[:1], dtype)[0]:            # 1.01 x m rounded to neither neighbour
        got[0] = lo[0]
    with pytest.raises(AssertionError, match="outside the tie band"):
        check_codes(got, v, np.abs(v), dtype)


def test_single_key_attention_operand_rounded_in_float32_passes():
    """One action row and no cached prefix: the attention output is the row's own bf16 V,
    copied into the 8 query heads of the one KV head, and the static scale is a bf16 max
    over 448; the quotients land on exact e4m3 midpoints.  Rounding them in float32 (the
    scale's reciprocal, then the product) flips some of them; the check accepts that."""
    dims = synth.chain_dims(layers=2, steps=2, M=1, prefix=0)
    wl = synth.workload4(dims)
    none = [np.zeros((0, dims["head_dim"]))] * dims["layers"]
    x0c, modc = synth.chain_inputs(dims, synth.CAL_SEED)
    sc = ref.calibrate(x0c, cp.oracle_weights(wl["layers"], "bf16"), none, none, modc, dims, 1e-6)
    tr = {}
    ref.chain(wl["x0"], cp.oracle_weights(wl["layers"], "e4m3"), sc, none, none, wl["mod"], dims, "e4m3",
              1e-6, trace=tr)
    o = tr[(0, 0)]["o"]
    v = o / sc[0][cp.SITE_O]
    v32 = (o.astype(np.float32) * (np.float32(1.0) / np.float32(sc[0][cp.SITE_O]))).astype(np.float64)
    got = codec.encode(v32, "e4m3")
    n, tot = check_codes(got, v, np.abs(o) / sc[0][cp.SITE_O], "e4m3")
    assert n > 0.01 * tot, "the case no longer lands on midpoints; the test lost its point"
