"""The allocation-free skinny GEMM (frt_skinny_gemm_splitk_noalloc) against the entry point
it varies (frt_skinny_gemm_splitk with a caller-provided partials workspace), through the
C ABI, on MI355X: the same kernels run on the same inputs, so the outputs must be equal
bit for bit.  Two calls in a row, the second with a smaller input, so the second reads a
scratch array that still holds the first call's partials.  Sizes beyond the scratch
array and the partials-only epilogue are refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import synth
from oracle import codec, ref

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def F():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X GPU")
    from gemm_chains_amd import device, frt
    frt.lib()
    return frt, device


def _inputs(frt, dev, M, N, K, dtype, layout, seed):
    dt = frt.DTYPES[dtype]
    w_bits = synth.weight_bf16(seed, 97, 1, K, N)
    wcodes, s_w, _ = ref.pack_weight_values(codec.bf16_decode(w_bits), None, dtype)
    a_val = synth.normal(seed, 97, 2, (M, K))
    acodes = synth.to_bf16_bits(a_val) if dtype == "bf16" else codec.e4m3_encode(a_val.astype(np.float64) * 60.0)
    a_pk = dev.to_dev(frt.frt_operand_pack_host(acodes, dt, M, K))
    w_pk = dev.to_dev(frt.frt_weight_pack_host(wcodes, dt, K, N, layout))
    cs = dev.to_dev(s_w.astype(np.float32)) if s_w is not None else None
    return dt, a_pk, w_pk, cs


def _pair(frt, dev, M, N, K, splits, dtype, epi):
    """(existing entry point's output, allocation-free entry point's output) as bytes."""
    layout = frt.W_GATE_UP if epi == frt.EPI_SILU_GATE_QUANT else frt.W_PLAIN
    dt, a_pk, w_pk, cs = _inputs(frt, dev, M, N, K, dtype, layout, seed=M + N + K + splits)
    act = 0.03125 if dtype == "e4m3" else 1.0
    out_scale = 0.0625 if dtype == "e4m3" else 1.0
    if epi == frt.EPI_SILU_GATE_QUANT:
        nbytes, odt = frt.frt_operand_bytes(dt, M, N // 2), dt
    else:
        nbytes, odt = M * N * 4, frt.F32
    outs = []
    for noalloc in (False, True):
        out = torch.full((nbytes,), 0xAB, dtype=torch.uint8, device="cuda")
        if noalloc:
            frt.frt_skinny_gemm_splitk_noalloc(M, N, K, splits, dt, layout, a_pk, w_pk, cs, act, epi, out, odt,
                                               out_scale)
        else:
            parts = torch.empty(splits * M * N, dtype=torch.float32, device="cuda")
            frt.frt_skinny_gemm_splitk(M, N, K, splits, dt, layout, a_pk, w_pk, cs, act, parts, parts.numel() * 4,
                                       epi, out, odt, out_scale)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    return outs


@pytest.mark.parametrize("dtype,epi_name", [("bf16", "EPI_STORE_F32"), ("e4m3", "EPI_SILU_GATE_QUANT"),
                                            ("bf16", "EPI_SILU_GATE_QUANT"), ("e4m3", "EPI_STORE_F32")])
def test_noalloc_matches_the_workspace_entry_point(F, dtype, epi_name):
    frt, dev = F
    epi = getattr(frt, epi_name)
    assert frt.frt_noalloc_scratch_bytes() == 16 << 20
    # first call: a large split (13.1 MB of partials at M = 50, N = 8192, s = 8 for bf16)
    big = (50, 8192, 1024, 8 if dtype == "bf16" else 2)
    small = (10, 1024, 1024, 2)
    for M, N, K, s in (big, small):
        ref_out, got = _pair(frt, dev, M, N, K, s, dtype, epi)
        assert np.array_equal(ref_out, got), f"{dtype} {epi_name} M={M} N={N} K={K} s={s}"
        print(f"no-alloc {dtype} {epi_name} M={M} N={N} K={K} s={s}: bit-identical", flush=True)


def test_noalloc_refuses_what_it_cannot_hold(F):
    frt, dev = F
    dt, a_pk, w_pk, cs = _inputs(frt, dev, 64, 16384, 2048, "bf16", frt.W_PLAIN, seed=3)
    out = torch.empty(64 * 16384 * 4, dtype=torch.uint8, device="cuda")
    with pytest.raises(frt.FrtError) as e:       # 8 x 64 x 16384 x 4 = 32 MiB of partials
        frt.frt_skinny_gemm_splitk_noalloc(64, 16384, 2048, 8, dt, frt.W_PLAIN, a_pk, w_pk, None, 1.0,
                                           frt.EPI_STORE_F32, out, frt.F32, 1.0)
    assert e.value.status == frt.E_WORKSPACE
    with pytest.raises(frt.FrtError) as e:       # the partials are the output: the caller owns them
        frt.frt_skinny_gemm_splitk_noalloc(64, 16384, 2048, 2, dt, frt.W_PLAIN, a_pk, w_pk, None, 1.0,
                                           frt.EPI_NONE, out, frt.F32, 1.0)
    assert e.value.status == frt.E_ARG
