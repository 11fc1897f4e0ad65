"""Pins of the oracle against what the pages and the mathematics fix (CPU only).

Each oracle function is checked against something other than itself:
  codecs      -> the format definitions (golden tables from the OCP FP8 and bfloat16
                 definitions), brute-force nearest-value search over every finite code
                 with ties to the even code, and torch's casts (library).
  RMSNorm     -> closed forms of the normalisation equation in the pages' graph-
                 simplification section (constant rows, mean(xhat^2) = ms/(ms+eps), the
                 [3, 4] row).
  gamma fold  -> (xhat * gamma) W == xhat (diag(gamma) W), exact on small integers.
  AdaRMSNorm  -> zero modulation reduces to RMSNorm; unit gate to a plain residual add.
  split-K     -> sum_j A_j W_j == A W exactly in float64 on small integers for every
                 split count, including one K-row per split.
  GEMM        -> triple loop.
  SiLU        -> SiLU(0) = 0, SiLU(x) - SiLU(-x) = x, torch's silu.
  attention   -> torch scaled_dot_product_attention in float64 with the KV head repeated,
                 equal keys giving the mean of V, one dominant logit selecting its V row.
  weight quant-> brute-force column maxima, power-of-two column scaling invariance.
  chain       -> composition of layer() calls; one layer equals the hand-composed
                 producer / GEMM / attention / consumer functions.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import codec, ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                c, v = line.split()
                rows.append((int(c, 16), float(v)))
    return rows


# ------------------------------------------------------------------ codecs

def _same(a, b):
    a, b = np.asarray(a, float), np.asarray(b, float)
    return np.all((a == b) & (np.signbit(a) == np.signbit(b)) | (np.isnan(a) & np.isnan(b)))


def test_e4m3_golden_values():
    rows = _read_golden("e4m3_ocp_values.txt")
    codes = np.array([c for c, _ in rows])
    vals = np.array([v for _, v in rows])
    assert _same(codec.e4m3_decode(codes), vals)
    fin = ~np.isnan(vals)
    assert np.array_equal(codec.e4m3_encode(vals[fin]), codes[fin].astype(np.uint8))


def test_bf16_golden_values():
    rows = _read_golden("bf16_values.txt")
    codes = np.array([c for c, _ in rows])
    vals = np.array([v for _, v in rows])
    assert _same(codec.bf16_decode(codes), vals)
    nonnan = ~np.isnan(vals)
    assert np.array_equal(codec.bf16_encode(vals[nonnan]), codes[nonnan].astype(np.uint16))


def _brute_nearest(values, table_codes, table_vals, sat_code=None, sat_at=None):
    """Nearest finite code by exhaustive search, ties to the even code; sign applied after."""
    a = np.abs(values)
    out = np.empty(a.shape, np.int64)
    for i, x in enumerate(a):
        if sat_at is not None and x >= sat_at:
            out[i] = sat_code
            continue
        d = np.abs(table_vals - x)
        best = np.flatnonzero(d == d.min())
        if len(best) > 1:
            best = [b for b in best if table_codes[b] % 2 == 0]
        out[i] = table_codes[best[0]]
    sign_bit = 0x80 if sat_code is not None and sat_code < 0x100 else 0x8000
    return np.where(np.signbit(values), out | sign_bit, out)


def _e4m3_table():
    codes = np.arange(0x7F)                   # 0x00 .. 0x7E, every finite non-negative code
    return codes, codec.e4m3_decode(codes)


def _e4m3_probe_values():
    codes, vals = _e4m3_table()
    mids = (vals[:-1] + vals[1:]) / 2
    pts = np.concatenate([vals, mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf),
                          [448.0, 456.0, 464.0, 470.0, 1e9, 2.0 ** -10, 2.0 ** -11, 1e-30]])
    rnd = np.random.default_rng(7)
    pts = np.concatenate([pts, np.exp(rnd.uniform(np.log(2.0 ** -12), np.log(600.0), 4000))])
    return np.concatenate([pts, -pts])


def test_fp4_golden_values():
    rows = _read_golden("fp4_e2m1_values.txt")
    codes = np.array([c for c, _ in rows])
    vals = np.array([v for _, v in rows])
    assert len(rows) == 16
    assert _same(codec.fp4_decode(codes), vals)
    assert np.array_equal(codec.fp4_encode(vals), codes.astype(np.uint8))


def _fp4_brute(v):
    """Nearest of the 8 E2M1 magnitudes by exhaustive search; ties to the even code
    (mantissa bit 0); beyond 6 the largest; the sign is copied."""
    mags = codec.fp4_decode(np.arange(8))
    out = []
    for x in np.asarray(v, float):
        a = abs(x)
        d = np.abs(mags - a)
        best = np.flatnonzero(d == d.min())
        c = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        out.append(c | (8 if np.signbit(x) else 0))
    return np.array(out, np.uint8)


def test_fp4_encode_matches_brute_force_nearest():
    mags = codec.fp4_decode(np.arange(8))
    mids = (mags[1:] + mags[:-1]) / 2
    g = np.random.default_rng(11)
    v = np.concatenate([mags, mids, np.nextafter(mids, 0), np.nextafter(mids, 10), [6.5, 7.99, 8.0, 1e9],
                        g.uniform(0, 9, 20000), g.standard_normal(20000) * 3])
    v = np.concatenate([v, -v])
    assert np.array_equal(codec.fp4_encode(v), _fp4_brute(v))


def test_mxfp4_block_scales():
    g = np.random.default_rng(12)
    w = g.standard_normal((128, 7)) * np.exp2(g.integers(-20, 20, (1, 7)))
    w[32:64, 3] = 0.0                                    # an all-zero block
    codes, sb, X = codec.mxfp4_encode(w)
    assert codes.shape == w.shape and sb.shape == (4, 7)
    amax = np.abs(w).reshape(4, 32, 7).max(axis=1)
    nz = amax > 0
    assert np.all(X == np.ldexp(1.0, sb.astype(int) - 127))          # E8M0: a power of two
    r = amax[nz] / X[nz]
    assert np.all((r >= 4.0) & (r < 8.0))                             # largest element exponent 2
    assert sb[1, 3] == 0 and np.all(codes[32:64, 3] == 0)
    # every element is the E2M1 rounding of w / X
    assert np.array_equal(codes, codec.fp4_encode(w / np.repeat(X, 32, axis=0)))
    dec = codec.mxfp4_decode(codes, sb)
    Xr = np.repeat(X, 32, axis=0)
    inside = np.abs(w) <= 6.0 * Xr
    assert np.all(np.abs(dec - w)[inside] <= Xr[inside])           # half the widest quantum (2 X)
    assert np.all(dec[~inside] == np.sign(w[~inside]) * 6.0 * Xr[~inside])  # (6X, 8X) saturates
    # scaling one block by 2**k leaves its codes and moves its scale byte by k
    w2 = w.copy()
    w2[64:96, 5] *= 2.0 ** 9
    c2, sb2, _ = codec.mxfp4_encode(w2)
    assert np.array_equal(c2, codes) and sb2[2, 5] == sb[2, 5] + 9
    assert np.array_equal(np.delete(sb2.ravel(), 2 * 7 + 5), np.delete(sb.ravel(), 2 * 7 + 5))


def test_e4m3_encode_matches_brute_force_nearest():
    codes, vals = _e4m3_table()
    v = _e4m3_probe_values()
    want = _brute_nearest(v, codes, vals, sat_code=0x7E, sat_at=448.0)
    got = codec.e4m3_encode(v).astype(np.int64)
    assert np.array_equal(got, want)


def test_e4m3_specials():
    assert codec.e4m3_encode([np.inf])[0] == 0x7E
    assert codec.e4m3_encode([-np.inf])[0] == 0xFE
    assert codec.e4m3_encode([np.nan])[0] == 0x7F
    assert codec.e4m3_encode([-0.0])[0] == 0x80
    assert codec.e4m3_encode([-1e-30])[0] == 0x80
    # decode(encode(x)) is the identity on every finite code
    c = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    assert np.array_equal(codec.e4m3_encode(codec.e4m3_decode(c)), c.astype(np.uint8))


def test_e4m3_matches_torch_cast_after_clamp():
    rnd = np.random.default_rng(11)
    v = np.concatenate([rnd.standard_normal(200000) * 60.0, _e4m3_probe_values()])
    v32 = v.astype(np.float32)                 # torch casts from float32; compare on those values
    clamped = np.clip(v32, -448.0, 448.0)
    t = torch.from_numpy(clamped).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codec.e4m3_encode(v32.astype(np.float64)), t)


def test_bf16_encode_matches_brute_force_nearest():
    codes = np.arange(0x7F80)                  # every finite non-negative bf16 code
    vals = codec.bf16_decode(codes)
    rnd = np.random.default_rng(3)
    pick = rnd.integers(0, 0x7F7F, 300)
    mids = (vals[pick] + vals[pick + 1]) / 2
    pts = np.concatenate([vals[pick], mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf),
                          np.exp(rnd.uniform(-90, 88, 300)), [2.0 ** -134, 3 * 2.0 ** -134]])
    pts = np.concatenate([pts, -pts])
    want = _brute_nearest(pts, codes, vals)
    assert np.array_equal(codec.bf16_encode(pts).astype(np.int64), want)


def test_bf16_overflow_and_specials():
    top = codec.bf16_decode(0x7F7F)
    half_ulp = 2.0 ** (127 - 8)
    assert codec.bf16_encode([top + half_ulp * 0.999])[0] == 0x7F7F
    assert codec.bf16_encode([top + half_ulp])[0] == 0x7F80     # tie goes to the even (infinite) side
    assert codec.bf16_encode([-np.inf])[0] == 0xFF80
    assert codec.bf16_encode([np.nan])[0] == 0x7FC0


def test_bf16_matches_torch_cast():
    rnd = np.random.default_rng(5)
    v = np.concatenate([rnd.standard_normal(100000) * 10.0 ** rnd.uniform(-30, 30, 100000),
                        rnd.standard_normal(1000) * 1e-39]).astype(np.float32)
    t = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(codec.bf16_encode(v.astype(np.float64)), t)


# ------------------------------------------------------------------ RMSNorm and folding

def test_rmsnorm_closed_forms():
    eps = 1e-6
    for c in (0.5, 3.0, -2.0):
        xh = ref.rms_normalise(np.full((1, 16), c), eps)
        assert np.allclose(xh, c / math.sqrt(c * c + eps), rtol=1e-15, atol=0)
    x = np.array([[3.0, 4.0]])
    assert np.allclose(ref.rms_normalise(x, eps), x / math.sqrt(12.5 + eps), rtol=1e-15, atol=0)
    rnd = np.random.default_rng(0)
    h = rnd.standard_normal((7, 1024)) * rnd.uniform(0.01, 10, (7, 1))
    ms = np.mean(h * h, axis=1)
    got = np.mean(ref.rms_normalise(h, eps) ** 2, axis=1)
    assert np.allclose(got, 1.0 - eps / (ms + eps), rtol=0, atol=1e-15)


def test_gamma_fold_equivalence():
    rnd = np.random.default_rng(1)
    xh = rnd.integers(-4, 5, (5, 12)).astype(float)
    g = rnd.integers(-3, 4, 12).astype(float)
    w = rnd.integers(-5, 6, (12, 9)).astype(float)
    assert np.array_equal((xh * g[None, :]) @ w, xh @ ref.fold_gamma(g, w))
    x = rnd.standard_normal((4, 64))
    g = 1 + 0.1 * rnd.standard_normal(64)
    w = rnd.standard_normal((64, 32))
    assert np.allclose(ref.rmsnorm_matmul(x, g, w, 1e-6),
                       ref.rms_normalise(x, 1e-6) @ ref.fold_gamma(g, w), rtol=1e-13, atol=1e-13)
    assert np.allclose(ref.rmsnorm_matmul(x, np.ones(64), w, 1e-6),
                       ref.rms_normalise(x, 1e-6) @ w, rtol=1e-15, atol=0)


def test_adarms_and_gate_special_cases():
    rnd = np.random.default_rng(2)
    r = rnd.standard_normal((3, 32))
    x = rnd.standard_normal((3, 32))
    z = np.zeros(32)
    out = ref.residual_norm_quant(r, x_parts=x[None], gate=np.ones(32), ada_scale=z,
                                  ada_shift=z, out_dtype="bf16")
    assert np.array_equal(out["h"], r + x)
    assert np.array_equal(out["y"], ref.rms_normalise(r + x, 1e-6))
    # scale only: y = xhat (1 + s); shift only: y = xhat + b
    s = rnd.standard_normal(32)
    out = ref.residual_norm_quant(r, ada_scale=s)
    assert np.allclose(out["y"], ref.rms_normalise(r, 1e-6) * (1 + s), rtol=1e-15, atol=0)
    out = ref.residual_norm_quant(r, ada_shift=s)
    assert np.allclose(out["y"], ref.rms_normalise(r, 1e-6) + s, rtol=1e-15, atol=1e-15)
    # gated residual on small integers with two partials and column scale
    parts = rnd.integers(-3, 4, (2, 3, 32)).astype(float)
    cs = rnd.integers(1, 4, 32).astype(float)
    g = rnd.integers(-2, 3, 32).astype(float)
    ri = rnd.integers(-5, 6, (3, 32)).astype(float)
    out = ref.residual_norm_quant(ri, x_parts=parts, x_colscale=cs, x_scale=2.0, gate=g)
    assert np.array_equal(out["h"], ri + g * ((parts[0] + parts[1]) * 2.0 * cs))
    # e4m3 output divides by the activation scale before rounding
    out = ref.residual_norm_quant(r, out_dtype="e4m3", act_scale=0.25)
    assert np.array_equal(out["v"], out["y"] / 0.25)
    assert np.array_equal(out["codes"], codec.e4m3_encode(out["y"] * 4.0))


# ------------------------------------------------------------------ GEMM and split-K

@pytest.mark.parametrize("K", [8, 24, 64])
def test_splitk_sum_is_exact_on_integers(K):
    rnd = np.random.default_rng(K)
    a = rnd.integers(-8, 9, (5, K)).astype(float)
    w = rnd.integers(-8, 9, (K, 7)).astype(float)
    full = a @ w
    for s in [d for d in range(1, K + 1) if K % d == 0]:
        p = ref.gemm_splitk(a, w, s)
        assert p.shape == (s, 5, 7)
        assert np.array_equal(ref.reduce_partials(p), full)


def test_gemm_matches_triple_loop():
    rnd = np.random.default_rng(4)
    a = rnd.standard_normal((3, 16))
    w = rnd.standard_normal((16, 5))
    c = np.zeros((3, 5))
    for i in range(3):
        for j in range(5):
            for k in range(16):
                c[i, j] += a[i, k] * w[k, j]
    p = ref.gemm_splitk(a, w, 4)
    assert np.allclose(ref.reduce_partials(p), c, rtol=1e-14, atol=1e-14)
    # chunk j covers rows [4j, 4j+4) of W
    assert np.allclose(p[2], a[:, 8:12] @ w[8:12, :], rtol=1e-15, atol=0)
    cs = rnd.uniform(0.5, 2, 5)
    assert np.allclose(ref.reduce_partials(p, 0.5, cs), c * 0.5 * cs[None, :], rtol=1e-14, atol=1e-14)


# ------------------------------------------------------------------ SiLU

def test_silu():
    assert ref.silu(np.array([0.0]))[0] == 0.0
    x = np.linspace(-30, 30, 1001)
    assert np.allclose(ref.silu(x) - ref.silu(-x), x, rtol=0, atol=1e-13)
    t = torch.nn.functional.silu(torch.from_numpy(x)).numpy()
    assert np.allclose(ref.silu(x), t, rtol=1e-15, atol=1e-15)
    c = np.concatenate([x[None, :100], x[None, 100:200]], axis=1)
    assert np.allclose(ref.silu_gate(c), ref.silu(x[:100]) * x[100:200], rtol=0, atol=0)


# ------------------------------------------------------------------ attention

def test_attention_matches_torch_sdpa():
    rnd = np.random.default_rng(6)
    M, nh, hd, T = 5, 4, 16, 37
    q = rnd.standard_normal((M, nh * hd))
    k = rnd.standard_normal((T, hd))
    v = rnd.standard_normal((T, hd))
    o, _ = ref.attention_prefix(q, k, v, nh, hd)
    qt = torch.from_numpy(q).reshape(M, nh, hd).transpose(0, 1)            # [nh][M][hd]
    kt = torch.from_numpy(k)[None].expand(nh, T, hd).contiguous()
    vt = torch.from_numpy(v)[None].expand(nh, T, hd).contiguous()
    want = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt).transpose(0, 1).reshape(M, nh * hd)
    assert np.allclose(o, want.numpy(), rtol=1e-12, atol=1e-12)


def test_attention_special_cases():
    rnd = np.random.default_rng(8)
    hd, T = 8, 10
    q = rnd.standard_normal((2, 2 * hd))
    k = np.tile(rnd.standard_normal((1, hd)), (T, 1))                     # all keys equal
    v = rnd.standard_normal((T, hd))
    o, _ = ref.attention_prefix(q, k, v, 2, hd)
    assert np.allclose(o, np.tile(v.mean(axis=0), 2)[None, :], rtol=1e-14, atol=1e-14)
    k = np.zeros((T, hd))
    k[3] = 100.0                                                           # one dominant logit
    q = np.ones((1, hd))
    o, _ = ref.attention_prefix(q, k, v, 1, hd)
    assert np.allclose(o[0], v[3], rtol=1e-12, atol=1e-12)


def test_attention_block_rounds_qkv_to_bf16_and_appends_own_rows():
    rnd = np.random.default_rng(9)
    M, nh, hd, P = 3, 2, 8, 5
    c = rnd.standard_normal((M, (nh + 2) * hd))
    kp = codec.bf16_round(rnd.standard_normal((P, hd)))
    vp = codec.bf16_round(rnd.standard_normal((P, hd)))
    out = ref.attention_block(c, kp, vp, nh, hd, "bf16")
    qb = codec.bf16_round(c[:, :nh * hd])
    kb = codec.bf16_round(c[:, nh * hd:nh * hd + hd])
    vb = codec.bf16_round(c[:, nh * hd + hd:])
    o, _ = ref.attention_prefix(qb, np.vstack([kp, kb]), np.vstack([vp, vb]), nh, hd)
    assert np.array_equal(out["o"], o)
    assert np.array_equal(out["codes"], codec.bf16_encode(o))


# ------------------------------------------------------------------ weight quantisation

def test_weight_quant_column_scales():
    rnd = np.random.default_rng(10)
    w = codec.bf16_round(rnd.standard_normal((64, 12)) / 8)
    w[:, 5] = 0.0
    codes, s_w, v = ref.pack_weight_values(w, None, "e4m3")
    for n in range(12):
        amax = max(abs(float(x)) for x in w[:, n])
        assert s_w[n] == float(np.float32(amax / 448.0))
    assert np.all(codes[:, 5] == 0) and s_w[5] == 0.0
    # the largest element of each non-zero column lands on +-448 (code 0x7E/0xFE)
    for n in [i for i in range(12) if i != 5]:
        k = int(np.argmax(np.abs(w[:, n])))
        assert codes[k, n] & 0x7F == 0x7E
    # scaling a column by 2^k leaves the codes unchanged and scales s_w by 2^k
    w2 = w.copy()
    w2[:, 3] *= 8.0
    codes2, s_w2, _ = ref.pack_weight_values(w2, None, "e4m3")
    assert np.array_equal(codes2, codes) and s_w2[3] == 8.0 * s_w[3]
    # gamma folding happens before quantisation
    g = rnd.uniform(0.5, 1.5, 64)
    c_g, s_g, _ = ref.pack_weight_values(w, g, "e4m3")
    c_f, s_f, _ = ref.pack_weight_values(g[:, None] * w, None, "e4m3")
    assert np.array_equal(c_g, c_f) and np.array_equal(s_g, s_f)
    cb, sb, _ = ref.pack_weight_values(w, g, "bf16")
    assert sb is None and np.array_equal(cb, codec.bf16_encode(g[:, None] * w))


# ------------------------------------------------------------------ layer / chain

def _tiny_chain_inputs(dtype, L=2, S=2):
    rnd = np.random.default_rng(12)
    dims = dict(n_heads=2, head_dim=8)
    M, H, F, P = 3, 16, 24, 5
    nqkv = (dims["n_heads"] + 2) * dims["head_dim"]
    weights = []
    for l in range(L):
        w = {}
        for name, (k, n) in dict(qkv=(H, nqkv), o=(dims["n_heads"] * dims["head_dim"], H),
                                 up=(H, 2 * F), down=(F, H)).items():
            codes, s_w, _ = ref.pack_weight_values(codec.bf16_round(rnd.standard_normal((k, n)) / math.sqrt(k)),
                                                   None, dtype)
            w[name] = codec.decode(codes, dtype)
            if s_w is not None:
                w["s" + name] = s_w
        weights.append(w)
    kp = [codec.bf16_round(rnd.standard_normal((P, 8))) for _ in range(L)]
    vp = [codec.bf16_round(rnd.standard_normal((P, 8))) for _ in range(L)]
    mod = rnd.standard_normal((S, L, 2, 3, H)) * 0.5
    x0 = rnd.standard_normal((M, H))
    scales = np.full((L, 4), 0.02)
    return x0, weights, scales, kp, vp, mod, dims


@pytest.mark.parametrize("dtype", ["bf16", "e4m3"])
def test_chain_is_composition_of_layers(dtype):
    x0, weights, scales, kp, vp, mod, dims = _tiny_chain_inputs(dtype)
    out = ref.chain(x0, weights, scales, kp, vp, mod, dims, dtype, 1e-6)
    h, xp, gp = x0, None, None
    for k in range(2):
        for l in range(2):
            h, xp, gp = ref.layer(h, xp, gp, mod[k, l, 0], mod[k, l, 1], weights[l], scales[l],
                                  kp[l], vp[l], dims, dtype, 1e-6)
    assert np.array_equal(out, h + gp[None, :] * xp)


@pytest.mark.parametrize("dtype", ["bf16", "e4m3"])
def test_one_layer_equals_hand_composed_steps(dtype):
    x0, weights, scales, kp, vp, mod, dims = _tiny_chain_inputs(dtype, L=1, S=1)
    w, sc = weights[0], scales[0]
    s = (lambda i: sc[i]) if dtype == "e4m3" else (lambda i: 1.0)
    nh, hd = dims["n_heads"], dims["head_dim"]
    p1 = ref.residual_norm_quant(x0, ada_scale=mod[0, 0, 0, 0], ada_shift=mod[0, 0, 0, 1],
                                 out_dtype=dtype, act_scale=s(0))
    c_qkv = ref.reduce_partials(ref.gemm_splitk(p1["deq"], w["qkv"], 2), s(0), w.get("sqkv"))
    att = ref.attention_block(c_qkv, kp[0], vp[0], nh, hd, dtype, s(1))
    o_parts = ref.gemm_splitk(att["deq"], w["o"], 1)
    p2 = ref.residual_norm_quant(p1["h"], x_parts=o_parts, x_colscale=w.get("so"), x_scale=s(1),
                                 gate=mod[0, 0, 0, 2], ada_scale=mod[0, 0, 1, 0],
                                 ada_shift=mod[0, 0, 1, 1], out_dtype=dtype, act_scale=s(2))
    c_up = ref.reduce_partials(ref.gemm_splitk(p2["deq"], w["up"], 1), s(2), w.get("sup"))
    z = ref.silu_gate_quant(c_up, dtype, s(3))
    d_parts = ref.gemm_splitk(z["deq"], w["down"], 3 if w["down"].shape[0] % 3 == 0 else 1)
    fin = ref.residual_norm_quant(p2["h"], x_parts=d_parts, x_colscale=w.get("sdown"), x_scale=s(3),
                                  gate=mod[0, 0, 1, 2])
    out = ref.chain(x0, weights, scales, kp, vp, mod, dims, dtype, 1e-6)
    assert np.allclose(out, fin["h"], rtol=1e-12, atol=1e-12)


def test_calibration_scales_cover_the_calibration_run():
    x0, weights, _, kp, vp, mod, dims = _tiny_chain_inputs("e4m3")
    sc = ref.calibrate(x0, weights, kp, vp, mod, dims, 1e-6)
    assert sc.shape == (2, 4) and np.all(sc > 0)
    # the first site of layer 0 sees AdaRMSNorm(x0) exactly: its amax sets the scale
    y = ref.ada_modulate(ref.rms_normalise(x0, 1e-6), mod[0, 0, 0, 0], mod[0, 0, 0, 1])
    assert sc[0, 0] >= float(np.float32(np.max(np.abs(y)) / 448.0))


def _calibration_by_hand(x0, weights, kp, vp, mod, nh, hd, eps):
    """The un-quantised chain walked element by element in plain Python (no oracle
    function but the pinned bf16 rounding of the stored Q, K, V): max |GEMM input| per
    (layer, site) over every flow step, over 448."""
    M, H = len(x0), len(x0[0])
    L, S, nq = len(weights), len(mod), nh * hd

    def matvec(row, W):
        return [sum(row[k] * W[k][n] for k in range(len(row))) for n in range(len(W[0]))]

    def ada(hrow, sc, sh):
        rms = math.sqrt(sum(v * v for v in hrow) / len(hrow) + eps)
        return [hrow[k] / rms * (1.0 + sc[k]) + sh[k] for k in range(len(hrow))]

    def b16(v):
        return float(codec.bf16_round(np.array([v]))[0])

    amax = [[0.0] * 4 for _ in range(L)]
    h = [[float(v) for v in row] for row in x0]
    x_prev = g_prev = None
    for s in range(S):
        for l in range(L):
            w = weights[l]
            if x_prev is not None:
                h = [[h[m][k] + g_prev[k] * x_prev[m][k] for k in range(H)] for m in range(M)]
            y = [ada(h[m], mod[s][l][0][0], mod[s][l][0][1]) for m in range(M)]
            amax[l][0] = max([amax[l][0]] + [abs(v) for r in y for v in r])
            c = [matvec(y[m], w["qkv"]) for m in range(M)]
            keys = [list(r) for r in kp[l]] + [[b16(c[m][nq + e]) for e in range(hd)] for m in range(M)]
            vals = [list(r) for r in vp[l]] + [[b16(c[m][nq + hd + e]) for e in range(hd)] for m in range(M)]
            o = [[0.0] * nq for _ in range(M)]
            for m in range(M):
                for hh in range(nh):
                    qv = [b16(c[m][hh * hd + e]) for e in range(hd)]
                    sc = [sum(qv[e] * kt[e] for e in range(hd)) / math.sqrt(hd) for kt in keys]
                    top = max(sc)
                    p = [math.exp(v - top) for v in sc]
                    for e in range(hd):
                        o[m][hh * hd + e] = sum(p[t] * vals[t][e] for t in range(len(p))) / sum(p)
            amax[l][1] = max([amax[l][1]] + [abs(v) for r in o for v in r])
            xa = [matvec(o[m], w["o"]) for m in range(M)]
            h = [[h[m][k] + mod[s][l][0][2][k] * xa[m][k] for k in range(H)] for m in range(M)]
            y2 = [ada(h[m], mod[s][l][1][0], mod[s][l][1][1]) for m in range(M)]
            amax[l][2] = max([amax[l][2]] + [abs(v) for r in y2 for v in r])
            F = len(w["up"][0]) // 2
            z = []
            for m in range(M):
                cu = matvec(y2[m], w["up"])
                z.append([cu[n] / (1.0 + math.exp(-cu[n])) * cu[F + n] for n in range(F)])
            amax[l][3] = max([amax[l][3]] + [abs(v) for r in z for v in r])
            x_prev = [matvec(z[m], w["down"]) for m in range(M)]
            g_prev = mod[s][l][1][2]
    return np.array(amax) / 448.0


def test_chain_calibration_matches_brute_force():
    """ref.calibrate on a tiny 2-layer x 2-step chain against the hand loop above.  The
    second flow step's modulation is larger, so every site's maximum comes from it (a
    calibration that looks at the first step only is caught), and the scales must be the
    float32 roundings of max/448 (OCP E4M3's largest finite value, not FNUZ's 240)."""
    x0, weights, _, kp, vp, mod, dims = _tiny_chain_inputs("bf16")
    master = [{n: w[n] for n in ("qkv", "o", "up", "down")} for w in weights]
    mod = mod.copy()
    mod[1] *= 3.0
    got = ref.calibrate(x0, master, kp, vp, mod, dims, 1e-6)
    want = _calibration_by_hand(x0.tolist(), [{n: w[n].tolist() for n in w} for w in master],
                                [k.tolist() for k in kp], [v.tolist() for v in vp], mod.tolist(),
                                dims["n_heads"], dims["head_dim"], 1e-6)
    first = _calibration_by_hand(x0.tolist(), [{n: w[n].tolist() for n in w} for w in master],
                                 [k.tolist() for k in kp], [v.tolist() for v in vp], mod[:1].tolist(),
                                 dims["n_heads"], dims["head_dim"], 1e-6)
    assert np.all(want > first * 1.01), "every site's maximum comes from the second step"
    assert got.shape == want.shape
    assert np.all(np.abs(got - want) <= 2.0 ** -23 * want + 1e-300)
    assert np.array_equal(got, got.astype(np.float32).astype(np.float64))


def test_block_calibration_is_the_largest_magnitude_over_448():
    # brute force on a tiny block: walk every element of the un-quantised run by hand
    rng = np.random.default_rng(5)
    M, K, F = 3, 8, 4
    r, x = rng.standard_normal((M, K)), rng.standard_normal((M, K))
    g, sc, sh = rng.standard_normal(K), 0.3 * rng.standard_normal(K), 0.3 * rng.standard_normal(K)
    w = rng.standard_normal((K, 2 * F)) / np.sqrt(K)
    s_y, s_z = ref.calibrate_block(r, x, g, sc, sh, w, 1e-6)
    big_y = big_z = 0.0
    for m in range(M):
        h = [r[m, k] + g[k] * x[m, k] for k in range(K)]
        rms = np.sqrt(sum(v * v for v in h) / K + 1e-6)
        y = [h[k] / rms * (1.0 + sc[k]) + sh[k] for k in range(K)]
        big_y = max(big_y, max(abs(v) for v in y))
        for n in range(F):
            gt = sum(y[k] * w[k, n] for k in range(K))
            up = sum(y[k] * w[k, F + n] for k in range(K))
            big_z = max(big_z, abs(gt / (1.0 + np.exp(-gt)) * up))
    assert s_y == float(np.float32(big_y / 448.0))
    assert abs(s_z - big_z / 448.0) <= 2.0 ** -23 * s_z + 1e-15


# ------------------------------------------------------------------ the pins catch planted mistakes

def _planted(monkeypatch, obj, name, fn, pin):
    with monkeypatch.context() as m:
        m.setattr(obj, name, fn)
        with pytest.raises((AssertionError, ValueError)):
            pin()


def test_pins_catch_planted_mistakes(monkeypatch):
    """Plausible mistakes planted in the oracle (on the CPU) each fail at least one pin."""
    np_ = np
    _planted(monkeypatch, ref, "rms_normalise",
             lambda h, eps: np_.asarray(h) / np_.sqrt(np_.mean(np_.asarray(h) ** 2, -1, keepdims=True)),
             test_rmsnorm_closed_forms)                                     # eps dropped
    _planted(monkeypatch, ref, "rms_normalise",
             lambda h, eps: np_.asarray(h) / (np_.sqrt(np_.mean(np_.asarray(h) ** 2, -1, keepdims=True)) + eps),
             test_rmsnorm_closed_forms)                                     # eps outside the root
    _planted(monkeypatch, ref, "fold_gamma",
             lambda g, w: np_.asarray(w) * np_.asarray(g)[None, : np_.asarray(w).shape[1]],
             test_gamma_fold_equivalence)                                   # scales columns
    _planted(monkeypatch, ref, "ada_modulate",
             lambda xh, sc, sh: np_.asarray(xh) * (1.0 if sc is None else np_.asarray(sc)[None, :])
             + (0.0 if sh is None else np_.asarray(sh)[None, :]),
             test_adarms_and_gate_special_cases)                            # scale without the 1+
    _planted(monkeypatch, ref, "silu", lambda g: np_.asarray(g) / (1.0 + np_.exp(np_.asarray(g))),
             test_silu)                                                     # sign of the exponent
    orig_split = ref.gemm_splitk

    def shifted(a, w, s):
        p = orig_split(a, w, s)
        return p[::-1].copy() if s > 1 else p
    _planted(monkeypatch, ref, "gemm_splitk", shifted, test_gemm_matches_triple_loop)  # chunk order
    orig_attn = ref.attention_prefix

    def no_scale(q, k, v, nh, hd):
        return orig_attn(np_.asarray(q) * np_.sqrt(hd), k, v, nh, hd)
    _planted(monkeypatch, ref, "attention_prefix", no_scale, test_attention_matches_torch_sdpa)
    orig_e = codec.e4m3_encode
    _planted(monkeypatch, codec, "e4m3_encode",
             lambda v: orig_e(np_.nextafter(np_.asarray(v, float), np_.sign(np_.asarray(v, float)) * np_.inf)),
             test_e4m3_encode_matches_brute_force_nearest)                  # ties away from zero
    orig_b = codec.bf16_encode
    _planted(monkeypatch, codec, "bf16_encode",
             lambda v: orig_b(np_.nextafter(np_.asarray(v, float), 0.0)),
             test_bf16_encode_matches_brute_force_nearest)                  # ties toward zero
    orig_f4 = codec.fp4_encode
    _planted(monkeypatch, codec, "fp4_encode",
             lambda v: orig_f4(np_.nextafter(np_.asarray(v, float), np_.sign(np_.asarray(v, float)) * np_.inf)),
             test_fp4_encode_matches_brute_force_nearest)                   # ties away from zero
    def mx_emax3(w):  # block exponent from the wrong element exponent (3 instead of 2)
        w = np_.asarray(w, float)
        K, N = w.shape
        b = w.reshape(K // 32, 32, N)
        amax = np_.abs(b).max(axis=1)
        nz = amax > 0
        e = np_.where(nz, np_.floor(np_.log2(np_.where(nz, amax, 1.0))) - 3, -127).astype(np_.int64)
        X = np_.ldexp(1.0, e)
        return codec.fp4_encode(b / X[:, None, :]).reshape(K, N), (e + 127).astype(np_.uint8), X
    _planted(monkeypatch, codec, "mxfp4_encode", mx_emax3, test_mxfp4_block_scales)
    with monkeypatch.context() as m:                                        # FNUZ's 240 for 448
        m.setattr(codec, "E4M3_MAX", 240.0)
        with pytest.raises(AssertionError):
            test_chain_calibration_matches_brute_force()
    orig_cal = ref.calibrate
    _planted(monkeypatch, ref, "calibrate",                                 # first flow step only
             lambda x0, w, kp, vp, mod, dims, eps: orig_cal(x0, w, kp, vp, np_.asarray(mod)[:1], dims, eps),
             test_chain_calibration_matches_brute_force)
    _planted(monkeypatch, ref, "calibrate",                                 # last layer's maxima for all
             lambda x0, w, kp, vp, mod, dims, eps: np_.repeat(orig_cal(x0, w, kp, vp, mod, dims, eps)[-1:],
                                                              len(w), axis=0),
             test_chain_calibration_matches_brute_force)
    orig_red = ref.reduce_partials
    _planted(monkeypatch, ref, "reduce_partials",
             lambda p, a=1.0, c=None: orig_red(np_.asarray(p)[:1], a, c),
             lambda: test_splitk_sum_is_exact_on_integers(24))               # drops partials
