"""GPU parity of each kernel against the oracle, through the C ABI (MI355X only).

Inputs are seeded and synthetic; both sides receive the same inputs (the oracle never
takes a GPU output as input).  Where an upstream float32 step feeds a rounding inside a
kernel, the inputs are chosen so that step is exact in float32 (dyadic values, power-of-
two scales), so the two sides round the same value.

Bars: codes bit-exact up to the tie band (tests/helpers.py); fp32 partial sums within
relative L2 1e-5 of the float64 products where the products are exact (bf16; e4m3 at
M <= 16, where the library multiplies the codes decoded to bf16) and 1e-4 through the
fp8 MFMA (e4m3 at M > 16: its internal sum keeps about 13 bits, ~1.5e-5 measured);
bf16 GEMM outputs within
relative L2 5e-3 and fp8 outputs within 2e-3 of the emulating oracle; split-K against
unsplit within 1e-5 (both on the GPU, in fp32: only the order of the k-step sums differs).
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import codec, ref
from tests.helpers import check_codes, e4m3_products_exact, partial_bar, rel_l2, silu_gate_mag

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("canaries")]


@pytest.fixture(scope="module")
def F():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X GPU")
    from gemm_chains_amd import frt, device
    frt.lib()  # raises if the HIP library is missing
    return frt, device


def _i16(a):
    return np.ascontiguousarray(a).view(np.int16)


def _u16(t):
    return t.cpu().numpy().view(np.uint16)


# ------------------------------------------------------------------ producer

PRODUCER_CASES = [
    # M, K, dtype, x_splits, gate, ada, colscale
    (10, 1024, "bf16", 0, False, False, False),      # plain RMSNorm of the residual (gamma folded)
    (10, 1024, "bf16", 4, True, True, False),
    (50, 1024, "bf16", 1, True, True, False),
    (50, 1024, "e4m3", 2, True, True, True),
    (10, 1024, "e4m3", 4, True, True, True),
    (64, 2048, "bf16", 8, True, False, False),
    (1, 128, "e4m3", 16, False, True, True),
    (17, 4096, "bf16", 3, True, True, False),
]


@pytest.mark.parametrize("M,K,dtype,splits,use_gate,use_ada,use_cs", PRODUCER_CASES)
def test_producer_parity(F, M, K, dtype, splits, use_gate, use_ada, use_cs):
    frt, dev = F
    dt = frt.DTYPES[dtype]
    seed = 1000 + M * 7 + K + splits
    r = synth.normal(seed, 90, 0, (M, K))
    parts = synth.normal(seed, 90, 1, (max(splits, 1), M, K)) if splits else None
    gate = synth.normal(seed, 90, 2, (K,)) if use_gate else None
    sc = synth.normal(seed, 90, 3, (K,), std=0.5) if use_ada else None
    sh = synth.normal(seed, 90, 4, (K,), std=0.5) if use_ada else None
    cs = np.abs(synth.normal(seed, 90, 5, (K,), std=0.01)) + np.float32(1e-3) if use_cs else None
    x_scale = np.float32(0.75)
    eps = 1e-6
    o0 = ref.residual_norm_quant(r, parts, cs, float(x_scale), gate, sc, sh, eps, dtype, 1.0)
    # a static scale that saturates the largest ~1% of values (tests the clamp)
    act = float(np.float32(np.quantile(np.abs(o0["y"]), 0.99) / 448.0)) if dtype == "e4m3" else 1.0
    o = ref.residual_norm_quant(r, parts, cs, float(x_scale), gate, sc, sh, eps, dtype, act)

    T = dev.to_dev
    h_out = dev.empty_f32(M, K)
    op = dev.empty_bytes(frt.frt_operand_bytes(dt, M, K))
    op.fill_(0xAB)
    frt.frt_residual_norm_quant(M, K, T(parts) if splits else None, splits if splits else 1, float(x_scale),
                                T(cs) if use_cs else None, T(r), h_out, T(gate) if use_gate else None,
                                T(sc) if use_ada else None, T(sh) if use_ada else None, eps, dt, act, op)
    torch.cuda.synchronize()
    h = dev.to_np(h_out)
    # float32 error bound of h = r + gate * (sum_j P_j) * x_scale * colscale: a few ulps of
    # the summands' magnitudes
    hmag = np.abs(r).astype(np.float64)
    if splits:
        xs_mag = np.sum(np.abs(parts.astype(np.float64)), axis=0) * float(x_scale)
        if use_cs:
            xs_mag = xs_mag * cs[None, :]
        if use_gate:
            xs_mag = xs_mag * np.abs(gate)[None, :]
        hmag = hmag + xs_mag
    assert np.all(np.abs(h - o["h"]) <= 2.0 ** -20 * hmag), "residual stream"
    Mp = 16 * math.ceil(M / 16)
    codes = dev.operand_codes(op, dt, Mp, K)
    check_codes(codes[:M], o["v"], o["mag"], dtype, label=f"producer {dtype} M={M}")
    assert np.all(codes[M:] == 0), "padding rows must hold zero codes"


def test_producer_inplace_and_residual_only(F):
    frt, dev = F
    M, K = 50, 1024
    r = synth.normal(5, 91, 0, (M, K))
    x = synth.normal(5, 91, 1, (2, M, K))
    g = synth.normal(5, 91, 2, (K,))
    o = ref.residual_norm_quant(r, x, None, 1.0, g, None, None, 1e-6, "bf16", 1.0)
    buf = dev.to_dev(r)
    frt.frt_residual_norm_quant(M, K, dev.to_dev(x), 2, 1.0, None, buf, buf, dev.to_dev(g), None, None, 1e-6,
                                frt.BF16, 1.0, None)
    torch.cuda.synchronize()
    assert np.allclose(dev.to_np(buf), o["h"], rtol=0, atol=1e-5)


# ------------------------------------------------------------------ weight packing

@pytest.mark.parametrize("K,N,dtype,layout,gamma", [
    (1024, 1024, "bf16", 0, True), (1024, 1024, "bf16", 0, False), (1024, 8192, "bf16", 1, False),
    (1024, 2560, "e4m3", 0, False), (4096, 1024, "e4m3", 0, False), (1024, 8192, "e4m3", 1, True),
    (2048, 16384, "e4m3", 1, False), (2048, 16384, "bf16", 1, True),
    (128, 48, "e4m3", 0, False), (32, 16, "bf16", 0, True)])
def test_pack_weight_parity(F, K, N, dtype, layout, gamma):
    frt, dev = F
    dt = frt.DTYPES[dtype]
    w = synth.weight_bf16(77, 92, K + N, K, N)
    if dtype == "e4m3" and N >= 48:
        w[:, 7] = 0                                  # an all-zero column: s_w = 0, zero codes
    g = synth.normal(77, 92, 1, (K,), std=0.1, mean=1.0) if gamma else None
    packed, cs = dev.pack_weight(w, dt, layout, gamma=g)
    torch.cuda.synchronize()
    codes = dev.weight_codes(packed, dt, K, N, layout)
    ocodes, s_w, v = ref.pack_weight_values(codec.bf16_decode(w), g, dtype)
    # the product gamma * W is exact in float64 and the kernel rounds W' (and W' / s_w)
    # once, as the oracle does: codes and column scales are bit-exact
    if dtype == "bf16":
        assert np.array_equal(codes, ocodes), f"{int(np.sum(codes != ocodes))} bf16 weight codes differ"
        if not gamma:
            assert np.array_equal(codes, w), "bf16 weights without gamma pack bit-exactly"
    else:
        gs = dev.to_np(cs).astype(np.float64)
        assert np.array_equal(gs, s_w), "column scales"
        assert np.array_equal(codes, ocodes), f"{int(np.sum(codes != ocodes))} e4m3 weight codes differ"
        if N >= 48:
            assert np.all(codes[:, 7] == 0) and gs[7] == 0.0


# ------------------------------------------------------------------ GEMM

def _gemm_inputs(frt, dev, M, N, K, dtype, seed, layout=0):
    """Oracle-prepared codes for A and W, host-packed into the GPU layout."""
    dt = frt.DTYPES[dtype]
    w_bits = synth.weight_bf16(seed, 93, 1, K, N)
    wcodes, s_w, _ = ref.pack_weight_values(codec.bf16_decode(w_bits), None, dtype)
    a_val = synth.normal(seed, 93, 2, (M, K))
    if dtype == "bf16":
        acodes = synth.to_bf16_bits(a_val)
    else:
        acodes = codec.e4m3_encode(a_val.astype(np.float64) * 60.0)
    a_pk = dev.to_dev(frt.frt_operand_pack_host(acodes, dt, M, K))
    w_pk = dev.to_dev(frt.frt_weight_pack_host(wcodes, dt, K, N, layout))
    a_dec = codec.decode(acodes, dtype)
    w_dec = codec.decode(wcodes, dtype)
    return dt, a_pk, w_pk, a_dec, w_dec, s_w


GEMM_CASES = [
    # M, N, K, dtype, splits
    (10, 1024, 1024, "bf16", 1), (10, 1024, 1024, "bf16", 2), (10, 1024, 1024, "bf16", 4),
    (50, 8192, 1024, "bf16", 1), (50, 8192, 1024, "bf16", 4), (50, 8192, 1024, "bf16", 8),
    (50, 1024, 4096, "bf16", 1), (50, 1024, 4096, "bf16", 4), (50, 1024, 4096, "bf16", 8),
    (10, 2560, 1024, "e4m3", 1), (10, 8192, 1024, "e4m3", 2), (10, 1024, 4096, "e4m3", 4),
    (50, 1280, 1024, "e4m3", 4), (64, 16384, 2048, "bf16", 2), (1, 16384, 2048, "e4m3", 4),
    (1, 16, 32, "bf16", 1), (17, 48, 96, "bf16", 1), (33, 32, 128, "e4m3", 1),
    (64, 64, 512, "bf16", 16), (49, 1024, 1024, "e4m3", 8),
    # either side of the e4m3 product switch: exact products up to 16 rows, the fp8 MFMA above
    (16, 2560, 1024, "e4m3", 2), (17, 1024, 1024, "e4m3", 1),
]


@pytest.mark.parametrize("M,N,K,dtype,splits", GEMM_CASES)
def test_gemm_partials_parity(F, M, N, K, dtype, splits):
    frt, dev = F
    dt, a_pk, w_pk, a_dec, w_dec, s_w = _gemm_inputs(frt, dev, M, N, K, dtype, seed=M * 31 + N + K)
    parts = dev.empty_f32(splits, M, N)
    frt.frt_skinny_gemm_splitk(M, N, K, splits, dt, frt.W_PLAIN, a_pk, w_pk, None, 1.0, parts,
                               parts.numel() * 4, frt.EPI_NONE, None, dt, 1.0)
    torch.cuda.synchronize()
    got = dev.to_np(parts)
    want = ref.gemm_splitk(a_dec, w_dec, splits)
    acc_bar = partial_bar(dtype, M)
    for j in range(splits):
        assert rel_l2(got[j], want[j]) <= acc_bar, f"partial {j}"


@pytest.mark.parametrize("M,N,K,dtype", [(10, 1024, 1024, "bf16"), (50, 1024, 4096, "e4m3"),
                                         (64, 16384, 2048, "e4m3"), (16, 2560, 1024, "bf16")])
def test_gemm_store_epilogues_and_splitk_invariance(F, M, N, K, dtype):
    frt, dev = F
    dt, a_pk, w_pk, a_dec, w_dec, s_w = _gemm_inputs(frt, dev, M, N, K, dtype, seed=7 + M + N)
    act = 0.03125 if dtype == "e4m3" else 1.0
    cs = dev.to_dev(s_w.astype(np.float32)) if dtype == "e4m3" else None
    c_o = ref.reduce_partials(ref.gemm_splitk(a_dec, w_dec, 1), act, s_w)
    g_mag = (np.abs(a_dec) @ np.abs(w_dec)) * act * (s_w[None, :] if s_w is not None else 1.0)
    outs = {}
    for s in (1, 2, 4):
        if (K // (32 if dtype == "bf16" else 128)) % s:
            continue
        parts = dev.empty_f32(s, M, N)
        c32 = dev.empty_f32(M, N)
        frt.frt_skinny_gemm_splitk(M, N, K, s, dt, frt.W_PLAIN, a_pk, w_pk, cs, act, parts, parts.numel() * 4,
                                   frt.EPI_STORE_F32, c32, frt.F32, 1.0)
        cb = dev.empty_bytes(M * N * 2).view(torch.int16).view(M, N)
        frt.frt_skinny_gemm_splitk(M, N, K, s, dt, frt.W_PLAIN, a_pk, w_pk, cs, act, parts, parts.numel() * 4,
                                   frt.EPI_STORE_BF16, cb, frt.BF16, 1.0)
        torch.cuda.synchronize()
        outs[s] = dev.to_np(c32)
        tol = 5e-3 if dtype == "bf16" else 2e-3
        assert rel_l2(outs[s], c_o) <= min(tol, partial_bar(dtype, M))
        bits = _u16(cb)
        assert rel_l2(codec.bf16_decode(bits), c_o) <= 5e-3
        # outputs of the fp8 MFMA carry its ~2^-16 internal rounding, so ~1% of their bf16
        # roundings sit within that error of a midpoint (all inside the tie band)
        frac = 0.01 if dtype == "bf16" or e4m3_products_exact(M) else 0.05
        check_codes(bits, c_o, g_mag, "bf16", max_frac=frac, label=f"bf16 store s={s}")
    for s in outs:
        assert rel_l2(outs[s], outs[1]) <= 1e-5, f"split {s} vs unsplit"
        print(f"split {s} vs unsplit rel L2 {rel_l2(outs[s], outs[1]):.2e}")


@pytest.mark.parametrize("M,N,K,dtype,splits", [(50, 8192, 1024, "bf16", 1), (50, 8192, 1024, "bf16", 4),
                                                (10, 8192, 1024, "e4m3", 1), (10, 8192, 1024, "e4m3", 2),
                                                (64, 256, 256, "bf16", 1), (3, 512, 128, "e4m3", 1)])
def test_gemm_silu_gate_epilogue(F, M, N, K, dtype, splits):
    frt, dev = F
    layout = frt.W_GATE_UP
    dt, a_pk, w_pk, a_dec, w_dec, s_w = _gemm_inputs(frt, dev, M, N, K, dtype, seed=11 + M + N, layout=layout)
    act = 0.015625 if dtype == "e4m3" else 1.0
    cs = dev.to_dev(s_w.astype(np.float32)) if dtype == "e4m3" else None
    c_o = ref.reduce_partials(ref.gemm_splitk(a_dec, w_dec, 1), act, s_w)
    n2 = N // 2
    out_scale = float(np.float32(np.quantile(np.abs(ref.silu_gate(c_o)), 0.995) / 448.0)) if dtype == "e4m3" else 1.0
    o = ref.silu_gate_quant(c_o, dtype, out_scale)
    mag = silu_gate_mag(c_o, a_dec, w_dec, act, s_w, dtype, out_scale)
    out = dev.empty_bytes(frt.frt_operand_bytes(dt, M, n2))
    out.fill_(0xCD)
    parts = dev.empty_f32(splits, M, N) if splits > 1 else None
    frt.frt_skinny_gemm_splitk(M, N, K, splits, dt, layout, a_pk, w_pk, cs, act, parts,
                               0 if parts is None else parts.numel() * 4, frt.EPI_SILU_GATE_QUANT, out, dt, out_scale)
    torch.cuda.synchronize()
    Mp = 16 * math.ceil(M / 16)
    codes = dev.operand_codes(out, dt, Mp, n2)
    check_codes(codes[:M], o["v"], mag, dtype, label=f"silu gate {dtype} s={splits}")
    assert np.all(codes[M:] == 0)


@pytest.mark.parametrize("M,N,K,dtype", [(50, 8192, 1024, "bf16"), (10, 1024, 4096, "bf16"), (17, 2560, 1024, "bf16"),
                                         (50, 1024, 1024, "e4m3")])
def test_gemm_results_ignore_operand_padding_rows(F, M, N, K, dtype):
    """The padding rows of a packed operand (rows M .. Mp-1) never reach a stored result:
    partials and the SiLU-gate output are bitwise the same whether those rows hold zero
    codes or other finite codes."""
    frt, dev = F
    dt = frt.DTYPES[dtype]
    Mp = 16 * math.ceil(M / 16)
    w_bits = synth.weight_bf16(5, 93, 1, K, N)
    wcodes, s_w, _ = ref.pack_weight_values(codec.bf16_decode(w_bits), None, dtype)
    a_val = synth.normal(5, 93, 2, (Mp, K))
    full = synth.to_bf16_bits(a_val) if dtype == "bf16" else codec.e4m3_encode(a_val.astype(np.float64) * 60.0)
    clean = dev.to_dev(frt.frt_operand_pack_host(full[:M], dt, M, K))      # padding rows: zero codes
    dirty = dev.to_dev(frt.frt_operand_pack_host(full, dt, Mp, K))         # padding rows: finite codes
    assert not torch.equal(clean, dirty)
    cs = dev.to_dev(s_w.astype(np.float32)) if dtype == "e4m3" else None
    act = 0.015625 if dtype == "e4m3" else 1.0
    out_scale = 0.05 if dtype == "e4m3" else 1.0
    got = {}
    for name, a_pk in (("clean", clean), ("dirty", dirty)):
        for layout, epi in ((frt.W_PLAIN, frt.EPI_NONE), (frt.W_GATE_UP, frt.EPI_SILU_GATE_QUANT)):
            w_pk = dev.to_dev(frt.frt_weight_pack_host(wcodes, dt, K, N, layout))
            if epi == frt.EPI_NONE:
                parts = dev.empty_f32(1, M, N)
                frt.frt_skinny_gemm_splitk(M, N, K, 1, dt, layout, a_pk, w_pk, None, 1.0, parts, parts.numel() * 4,
                                           epi, None, dt, 1.0)
                torch.cuda.synchronize()
                got[name, epi] = dev.to_np(parts)
            else:
                out = dev.empty_bytes(frt.frt_operand_bytes(dt, M, N // 2))
                out.fill_(0xCD)
                frt.frt_skinny_gemm_splitk(M, N, K, 1, dt, layout, a_pk, w_pk, cs, act, None, 0, epi, out, dt,
                                           out_scale)
                torch.cuda.synchronize()
                got[name, epi] = out.cpu().numpy()
    for epi in (frt.EPI_NONE, frt.EPI_SILU_GATE_QUANT):
        assert np.array_equal(got["clean", epi], got["dirty", epi]), f"epilogue {epi}"


# ------------------------------------------------------------------ fused QKV GEMM

@pytest.mark.parametrize("M,K,dtype,splits", [(50, 1024, "bf16", 1), (50, 1024, "bf16", 4), (10, 1024, "e4m3", 1),
                                              (10, 1024, "e4m3", 2), (64, 2048, "bf16", 2), (1, 128, "e4m3", 1)])
def test_qkv_gemm_epilogue(F, M, K, dtype, splits):
    frt, dev = F
    nh, hd = 8, 128
    N = (nh + 2) * hd
    dt, a_pk, w_pk, a_dec, w_dec, s_w = _gemm_inputs(frt, dev, M, N, K, dtype, seed=21 + M + K)
    act = 0.0625 if dtype == "e4m3" else 1.0
    cs = dev.to_dev(s_w.astype(np.float32)) if dtype == "e4m3" else None
    c_o = ref.reduce_partials(ref.gemm_splitk(a_dec, w_dec, 1), act, s_w)
    g_mag = (np.abs(a_dec) @ np.abs(w_dec)) * act * (s_w[None, :] if s_w is not None else 1.0)
    qo = dev.empty_bytes(M * nh * hd * 2).view(torch.int16).view(M, nh * hd)
    kc = dev.empty_bytes((M + 3) * hd * 2).view(torch.int16).view(M + 3, hd).zero_()   # rows 3.. as in a key cache
    ldv = (M + 3 + 31) // 32 * 32
    vc = dev.empty_bytes(hd * ldv * 2).view(torch.int16).view(hd, ldv).zero_()         # transposed value cache
    parts = dev.empty_f32(splits, M, N) if splits > 1 else None
    frt.frt_skinny_gemm_qkv(M, K, nh, hd, splits, dt, a_pk, w_pk, cs, act, parts,
                            0 if parts is None else parts.numel() * 4, qo, kc[3:], vc[:, 3:], ldv)
    torch.cuda.synchronize()
    got = np.concatenate([_u16(qo), _u16(kc[3:]), _u16(vc[:, 3:3 + M]).T], axis=1)
    frac = 0.01 if dtype == "bf16" or e4m3_products_exact(M) else 0.05
    check_codes(got, c_o, g_mag, "bf16", max_frac=frac, label=f"qkv {dtype} s={splits}")
    assert np.all(_u16(kc[:3]) == 0) and np.all(_u16(vc[:, :3]) == 0) and np.all(_u16(vc[:, 3 + M:]) == 0), \
        "cache entries outside the own rows are left untouched"


# ------------------------------------------------------------------ attention

@pytest.mark.parametrize("M,out_dtype,prefix", [(50, "bf16", 800), (10, "e4m3", 800), (50, "e4m3", 800),
                                                (1, "bf16", 0), (64, "bf16", 37), (17, "bf16", 800),
                                                (50, "bf16", 2000), (10, "bf16", 127), (3, "bf16", 8190)])
def test_attention_parity(F, M, out_dtype, prefix):
    frt, dev = F
    nh, hd = 8, 128
    T = prefix + M
    dt = frt.DTYPES[out_dtype]
    qb = synth.to_bf16_bits(synth.normal(M + prefix, 94, 0, (M, nh * hd)))
    kb = synth.to_bf16_bits(synth.normal(M + prefix, 94, 1, (T, hd)))
    vb = synth.to_bf16_bits(synth.normal(M + prefix, 94, 2, (T, hd)))
    o, mag = ref.attention_prefix(codec.bf16_decode(qb), codec.bf16_decode(kb), codec.bf16_decode(vb), nh, hd)
    out_scale = float(np.float32(np.max(np.abs(o)) / 448.0)) if out_dtype == "e4m3" else 1.0
    v, _, _ = ref.quantise(o, out_dtype, out_scale)
    if out_dtype == "e4m3":
        mag = mag / out_scale
    wsb = frt.frt_attention_workspace_bytes(M, nh, hd, T)
    ws = dev.empty_bytes(wsb)
    ws.fill_(0x7F)                                                    # no initial contents needed
    ldv = (T + 31) // 32 * 32
    vt = np.full((hd, ldv), 0x7FC0, np.uint16)                        # padding holds NaN: never used
    vt[:, :T] = vb.T
    ops = []
    for _ in range(2):                       # the second call reuses the workspace as left by the first
        op = dev.empty_bytes(frt.frt_operand_bytes(dt, M, nh * hd))
        op.fill_(0xAB)
        frt.frt_attention_prefix(M, nh, hd, T, dev.to_dev(_i16(qb)), dev.to_dev(_i16(kb)), dev.to_dev(_i16(vt)),
                                 ldv, dt, out_scale, op, ws, wsb)
        ops.append(op)
    torch.cuda.synchronize()
    Mp = 16 * math.ceil(M / 16)
    codes = dev.operand_codes(ops[0], dt, Mp, nh * hd)
    check_codes(codes[:M], v, mag, out_dtype, label=f"attention {out_dtype} M={M} T={T}")
    assert np.all(codes[M:] == 0)
    assert torch.equal(ops[0], ops[1]), "repeat call must be bit-identical"
