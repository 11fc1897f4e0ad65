"""GPU parity of the 4-bit weight path (OCP MXFP4 weights x e4m3 activations) against
the oracle, through the C ABI (MI355X only).

- Packing: the kernel forms gamma * W exactly in float64, picks each 32-element block's
  E8M0 exponent and rounds every element once, as the oracle does, so codes and scale
  bytes are bit-exact; hand-made blocks pin the FP4 tie and saturation rules, an all-zero
  block and the exponent clamp.
- GEMM: FP4 x FP8 products are exact and the block scales are powers of two, but the
  block-scaled MFMA sums its products inside the instruction with less than fp32
  precision (about 1.5e-5 relative measured), so the float32 partials are held to
  relative L2 1e-4 of the float64 products of the decoded values.  The weights' per-block magnitudes differ by
  up to 2^12, so a block paired with the wrong scale or the wrong activations is far
  outside that bar.
- Epilogues (store, SiLU-gate quantisation, fused QKV scatter) run on the same sums:
  their codes are checked up to the tie band, teacher-forced from the oracle's sums.
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import codec, ref
from tests.helpers import check_codes, rel_l2, silu_gate_mag

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("canaries")]


@pytest.fixture(scope="module")
def F():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X GPU")
    from gemm_chains_amd import frt, device
    frt.lib()  # raises if the HIP library is missing
    return frt, device


def _bits(values):
    """Exactly representable float values -> bf16 bit patterns (truncation is exact here)."""
    return (np.asarray(values, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _hand_blocks(w):
    """Overwrite a few blocks with values that pin the FP4 rounding rules (bf16-exact).

    Column 3, block 0: amax 6, so X = 1 and every midpoint of the FP4 grid is hit exactly
    (ties go to the even code); block 1: amax 7.5 -> X = 1 and 7.5 saturates to 6.
    Column 5, block 2: all zero -> scale byte 0, zero codes.  Column 6, block 0: amax
    2^-130 -> exponent clamped to -127.
    """
    mids = [6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0,
            0.0, -0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 5.5, 4.5, 0.125, 0.375, 2.25, 2.75, 1.125, 1.375, -6.0]
    w[0:32, 3] = _bits(mids)
    w[32:64, 3] = _bits([7.5] + [0.5 * i for i in range(-15, 16)])
    w[64:96, 5] = 0
    w[0:32, 6] = 0
    w[0, 6] = 0x0008                      # 2^-130 (bf16 subnormal)
    w[1, 6] = 0x8004                      # -2^-131
    return w


@pytest.mark.parametrize("K,N,layout,gamma", [(256, 64, 0, False), (256, 64, 0, True), (512, 256, 1, False),
                                              (1024, 2560, 0, True), (2048, 16384, 1, False), (128, 16, 0, False)])
def test_mxfp4_pack_parity(F, K, N, layout, gamma):
    frt, dev = F
    w = synth.weight_bf16_block_spread(78, 96, K + N, K, N)
    if N >= 16 and K >= 128:
        w = _hand_blocks(w)
    g = synth.normal(78, 96, 2, (K,), std=0.1, mean=1.0) if gamma else None
    packed, cs = dev.pack_weight(w, frt.MXFP4, layout, gamma=g)
    torch.cuda.synchronize()
    assert cs is None and packed.numel() == K * N // 2 + K * N // 32
    codes, sb = frt.frt_weight_unpack_mxfp4_host(dev.to_np(packed), K, N, layout)
    ocodes, osb, _ = ref.pack_weight_mxfp4(codec.bf16_decode(w), g)
    assert np.array_equal(sb, osb), f"{int(np.sum(sb != osb))} scale bytes differ"
    assert np.array_equal(codes, ocodes), f"{int(np.sum(codes != ocodes))} FP4 codes differ"
    if not gamma:
        # the hand-made blocks, against values read off the FP4 E2M1 grid
        assert sb[0, 3] == 127 and sb[1, 3] == 127 and sb[2, 5] == 0 and sb[0, 6] == 0
        want = [7, 0, 2, 2, 4, 4, 6, 6, 8, 10, 10, 12, 12, 14, 14, 0, 8, 1, 2, 3, 4, 5, 6, 7, 6, 0, 1, 4, 5, 2, 3, 15]
        assert codes[0:32, 3].tolist() == want
        assert codes[32, 3] == 7
        assert np.all(codes[64:96, 5] == 0)
        assert codes[0, 6] == 0 and codes[1, 6] == 8   # 2^-3 and -2^-4 of the clamped scale round to 0


def _mx_inputs(frt, dev, M, N, K, seed, layout=0):
    """Oracle-prepared e4m3 activation codes and MXFP4 weights, host-packed for the GPU."""
    w_bits = synth.weight_bf16_block_spread(seed, 97, 1, K, N)
    wcodes, sb, w_dec = ref.pack_weight_mxfp4(codec.bf16_decode(w_bits))
    acodes = codec.e4m3_encode(synth.normal(seed, 97, 2, (M, K)).astype(np.float64) * 60.0)
    a_pk = dev.to_dev(frt.frt_operand_pack_host(acodes, frt.E4M3, M, K))
    w_pk = dev.to_dev(frt.frt_weight_pack_mxfp4_host(wcodes, sb, K, N, layout))
    return a_pk, w_pk, codec.e4m3_decode(acodes), w_dec


MX_GEMM_CASES = [
    # M, N, K, splits
    (10, 2560, 1024, 1), (10, 1024, 1024, 4), (50, 1024, 4096, 4), (50, 8192, 1024, 1),
    (50, 16384, 2048, 2), (64, 16384, 2048, 4), (1, 16384, 2048, 4), (33, 32, 128, 1),
    (17, 48, 256, 2), (49, 1024, 1024, 8), (64, 64, 2048, 16),
]


@pytest.mark.parametrize("M,N,K,splits", MX_GEMM_CASES)
def test_mxfp4_gemm_partials_parity(F, M, N, K, splits):
    frt, dev = F
    a_pk, w_pk, a_dec, w_dec = _mx_inputs(frt, dev, M, N, K, seed=M * 31 + N + K)
    parts = dev.empty_f32(splits, M, N)
    frt.frt_skinny_gemm_splitk(M, N, K, splits, frt.MXFP4, frt.W_PLAIN, a_pk, w_pk, None, 1.0, parts,
                               parts.numel() * 4, frt.EPI_NONE, None, frt.E4M3, 1.0)
    torch.cuda.synchronize()
    got = dev.to_np(parts)
    want = ref.gemm_splitk(a_dec, w_dec, splits)
    for j in range(splits):
        e = rel_l2(got[j], want[j])
        assert e <= 1e-4, f"partial {j}: rel L2 {e:.3e}"


@pytest.mark.parametrize("M,N,K", [(10, 1024, 1024), (50, 1024, 4096), (64, 16384, 2048)])
def test_mxfp4_gemm_store_and_splitk_invariance(F, M, N, K):
    frt, dev = F
    a_pk, w_pk, a_dec, w_dec = _mx_inputs(frt, dev, M, N, K, seed=7 + M + N)
    act = 0.03125
    c_o = ref.reduce_partials(ref.gemm_splitk(a_dec, w_dec, 1), act, None)
    g_mag = (np.abs(a_dec) @ np.abs(w_dec)) * act
    outs = {}
    for s in (1, 2, 4):
        parts = dev.empty_f32(s, M, N)
        c32 = dev.empty_f32(M, N)
        frt.frt_skinny_gemm_splitk(M, N, K, s, frt.MXFP4, frt.W_PLAIN, a_pk, w_pk, None, act, parts,
                                   parts.numel() * 4, frt.EPI_STORE_F32, c32, frt.F32, 1.0)
        cb = dev.empty_bytes(M * N * 2).view(torch.int16).view(M, N)
        frt.frt_skinny_gemm_splitk(M, N, K, s, frt.MXFP4, frt.W_PLAIN, a_pk, w_pk, None, act, parts,
                                   parts.numel() * 4, frt.EPI_STORE_BF16, cb, frt.BF16, 1.0)
        torch.cuda.synchronize()
        outs[s] = dev.to_np(c32)
        assert rel_l2(outs[s], c_o) <= 1e-4
        check_codes(cb.cpu().numpy().view(np.uint16), c_o, g_mag, "bf16", max_frac=0.05, label=f"bf16 store s={s}")
    for s in outs:
        assert rel_l2(outs[s], outs[1]) <= 1e-5, f"split {s} vs unsplit"


@pytest.mark.parametrize("M,N,K,splits", [(10, 8192, 1024, 1), (50, 8192, 1024, 1), (50, 8192, 1024, 2),
                                          (64, 32768, 2048, 1), (3, 512, 128, 1)])
def test_mxfp4_gemm_silu_gate_epilogue(F, M, N, K, splits):
    frt, dev = F
    layout = frt.W_GATE_UP
    a_pk, w_pk, a_dec, w_dec = _mx_inputs(frt, dev, M, N, K, seed=11 + M + N, layout=layout)
    act = 0.015625
    c_o = ref.reduce_partials(ref.gemm_splitk(a_dec, w_dec, 1), act, None)
    n2 = N // 2
    out_scale = float(np.float32(np.quantile(np.abs(ref.silu_gate(c_o)), 0.995) / 448.0))
    o = ref.silu_gate_quant(c_o, "e4m3", out_scale)
    mag = silu_gate_mag(c_o, a_dec, w_dec, act, None, "e4m3", out_scale)
    out = dev.empty_bytes(frt.frt_operand_bytes(frt.E4M3, M, n2))
    out.fill_(0xCD)
    parts = dev.empty_f32(splits, M, N) if splits > 1 else None
    frt.frt_skinny_gemm_splitk(M, N, K, splits, frt.MXFP4, layout, a_pk, w_pk, None, act, parts,
                               0 if parts is None else parts.numel() * 4, frt.EPI_SILU_GATE_QUANT, out, frt.E4M3,
                               out_scale)
    torch.cuda.synchronize()
    Mp = 16 * math.ceil(M / 16)
    codes = dev.operand_codes(out, frt.E4M3, Mp, n2)
    check_codes(codes[:M], o["v"], mag, "e4m3", label=f"silu gate mxfp4 s={splits}")
    assert np.all(codes[M:] == 0)


@pytest.mark.parametrize("M,K,splits", [(10, 1024, 1), (50, 1024, 2), (1, 128, 1)])
def test_mxfp4_qkv_gemm_epilogue(F, M, K, splits):
    frt, dev = F
    nh, hd = 8, 128
    N = (nh + 2) * hd
    a_pk, w_pk, a_dec, w_dec = _mx_inputs(frt, dev, M, N, K, seed=21 + M + K)
    act = 0.0625
    c_o = ref.reduce_partials(ref.gemm_splitk(a_dec, w_dec, 1), act, None)
    g_mag = (np.abs(a_dec) @ np.abs(w_dec)) * act
    qo = dev.empty_bytes(M * nh * hd * 2).view(torch.int16).view(M, nh * hd).zero_()
    kc = dev.empty_bytes(M * hd * 2).view(torch.int16).view(M, hd).zero_()
    ldv = (M + 31) // 32 * 32
    vc = dev.empty_bytes(hd * ldv * 2).view(torch.int16).view(hd, ldv).zero_()
    parts = dev.empty_f32(splits, M, N) if splits > 1 else None
    frt.frt_skinny_gemm_qkv(M, K, nh, hd, splits, frt.MXFP4, a_pk, w_pk, None, act, parts,
                            0 if parts is None else parts.numel() * 4, qo, kc, vc, ldv)
    torch.cuda.synchronize()
    u16 = lambda t: t.cpu().numpy().view(np.uint16)
    got = np.concatenate([u16(qo), u16(kc), u16(vc[:, :M]).T], axis=1)
    check_codes(got, c_o, g_mag, "bf16", max_frac=0.05, label=f"qkv mxfp4 s={splits}")
