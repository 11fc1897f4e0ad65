"""GPU parity of the whole action-decoder chain against the oracle (MI355X only).

Both sides start from the same seeded inputs and bf16 master weights; each quantises the
weights itself (the packing kernel's codes are checked in test_gpu_kernels.py).  Static
activation scales come from the oracle's calibration run and are given to both sides.

Two gates, both required:

- Teacher-forced, per (flow step, layer): a chain built with debug buffers keeps every
  kernel's inputs and outputs; each kernel of each layer-step is compared with the
  oracle's step computed from the GPU's own inputs to it, at the per-kernel bars
  (tests/chain_parity.py): residual streams within 2^-20 of their summands, every GEMM
  input's codes within the tie band, fp32 partials within 1e-5 where the products are
  exact (bf16; e4m3 at M <= 16) / 1e-4 (the fp8 and FP4 x FP8 MFMAs) of the float64
  products.  A wiring mistake at any layer-step fails here at kernel
  tolerance.
- End to end: the final residual stream against the oracle chain run free.  Single
  rounding flips that the tie band allows are amplified by later layers, so this bar is
  twice the oracle's own sensitivity: the largest change of the oracle's output over
  three reruns with every GEMM input perturbed by relative noise before rounding (2^-22,
  a few fp32 ulps, for bf16; 2^-17, the tie band's width, for e4m3).

The production chain (graph replay, weight read-ahead, attention merge fused into the O
projection) must equal the debug chain bit for bit, graph replay must equal eager
launches, and two replays must agree (the pages' state-reuse result keeps outputs
bit-identical; replay reuses the same arguments and addresses).
"""
import time

import numpy as np
import pytest
import torch

import synth
from oracle import codec, ref
from tests import chain_parity as cp
from tests.helpers import record, rel_l2

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def F():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X GPU")
    from gemm_chains_amd import chain, frt
    frt.lib()
    return frt, chain


def _prefixes(wl):
    return ([codec.bf16_decode(l["k_prefix"]) for l in wl["layers"]],
            [codec.bf16_decode(l["v_prefix"]) for l in wl["layers"]])


def _oracle_scales(wl, dims):
    kp, vp = _prefixes(wl)
    x0c, modc = synth.chain_inputs(dims, synth.CAL_SEED)
    return ref.calibrate(x0c, cp.oracle_weights(wl["layers"], "bf16"), kp, vp, modc, dims, 1e-6)


def _oracle_and_bar(wl, ws, scales, adt, seeds=(95, 96, 97)):
    """The oracle chain's output and the end-to-end bar (2x its own sensitivity)."""
    kp, vp = _prefixes(wl)
    dims = wl["dims"]
    sc = scales if scales is not None else np.ones((dims["layers"], 4))

    def run(perturb=None):
        return ref.chain(wl["x0"], ws, sc, kp, vp, wl["mod"], dims, adt, 1e-6, perturb=perturb)
    want = run()
    noise = 2.0 ** -22 if adt == "bf16" else 2.0 ** -17
    sens = cp.sensitivity(run, want, noise, seeds)
    return want, sens, 2.0 * max(sens, 1e-7)


def _figs(worst, err, sens):
    return (f"teacher-forced residual {worst['h']:.1e}, partials {max(worst['p_o'], worst['p_down']):.1e}, "
            f"codes off {100 * worst['code_frac']:.2f} %; end to end {err:.3e} (oracle sensitivity {sens:.3e})")


def _run(chain, dims, packed, wl, scales, **kw):
    ch = chain.Chain(dims, packed, **kw)
    chain.load_workload(ch, wl, scales)
    ch.run()
    torch.cuda.synchronize()
    return ch


@pytest.mark.parametrize("wdtype,M,splits", [("bf16", 50, (0, 0, 0, 0)), ("e4m3", 50, (0, 0, 0, 0)),
                                             ("bf16", 10, (2, 1, 2, 8)), ("e4m3", 10, (1, 2, 1, 4)),
                                             ("mxfp4", 50, (0, 0, 0, 0)), ("mxfp4", 10, (1, 2, 1, 4)),
                                             ("bf16", 10, (0, 0, 0, 0)), ("e4m3", 10, (0, 0, 0, 0))])
def test_chain_parity(F, wdtype, M, splits):
    frt, chain = F
    dims = synth.chain_dims(layers=2, steps=2, M=M)
    wl = synth.workload4(dims)
    ws = cp.oracle_weights(wl["layers"], wdtype)
    adt = "bf16" if wdtype == "bf16" else "e4m3"   # MXFP4 weights multiply e4m3 activations
    scales = _oracle_scales(wl, dims) if adt == "e4m3" else None
    want, sens, bar = _oracle_and_bar(wl, ws, scales, adt)
    kp, vp = _prefixes(wl)

    packed = chain.PackedLayers(wl["layers"], dims, frt.DTYPES[wdtype])
    cg = _run(chain, dims, packed, wl, scales, splits=splits, use_graph=True, keep_intermediates=True)
    d = cp.gpu_dumps(frt, cg, dims, frt.DTYPES[wdtype])
    worst = cp.teacher_forced_check(d, wl["x0"], wl["mod"], kp, vp, ws, scales, dims, adt,
                                    wdtype=wdtype)
    got = d["x_out"]
    err = rel_l2(got, want)
    log(f"chain {wdtype} M={M} splits={splits}: teacher-forced worst {worst}; end to end rel L2 {err:.3e}, "
        f"oracle sensitivity {sens:.3e}, bar {bar:.3e}, kernels {cg.kernel_count()}")
    record(f"chain 2x2 {wdtype} M={M} splits={splits}", _figs(worst, err, sens))
    assert err <= bar
    # replay twice: bit-identical; eager launches of the production chain: bit-identical
    cg.run()
    torch.cuda.synchronize()
    assert np.array_equal(cg.read("x_out").reshape(M, -1), got)
    ce = _run(chain, dims, packed, wl, scales, splits=splits, use_graph=False, keep_intermediates=False)
    # without debug buffers the attention merge runs inside the O projection (one kernel
    # fewer per layer when the library picks the O split); the sums are bitwise the same
    assert np.array_equal(ce.read("x_out").reshape(M, -1), got), "eager production chain vs debug graph"
    fused = splits[1] == 0
    assert ce.kernel_count() == cg.kernel_count() - dims["steps"] * dims["layers"] * (1 + fused)
    cg.close()
    ce.close()


@pytest.mark.parametrize("M,prefix,wdtype", [(1, 0, "bf16"), (64, 100, "bf16"), (17, 300, "bf16"), (50, 0, "bf16"),
                                             (1, 0, "e4m3"), (64, 100, "mxfp4"), (17, 300, "e4m3"), (33, 31, "mxfp4"),
                                             (50, 1100, "bf16"), (10, 900, "e4m3"), (10, 1000, "mxfp4"),
                                             (10, 1100, "bf16")])
def test_chain_edge_shapes(F, M, prefix, wdtype):
    """Smallest and largest action chunks and short prefixes: no prefix (one key chunk,
    the merge kernel not needed), and prefixes that give 2..4 chunks (merge fused into
    the O projection), in bf16, e4m3 and MXFP4 weights; longer prefixes that give 9, 15
    and 16 key chunks (the fused merge's record slots: one per chunk up to 15, then 16),
    and 18 chunks (past what the fused merge takes: chunks, a merge kernel, the O GEMM);
    teacher-forced and end to end against the oracle; the production chain (fused,
    read-ahead on) must equal the debug chain bit for bit."""
    frt, chain = F
    dims = synth.chain_dims(layers=2, steps=2, M=M, prefix=prefix)
    wl = synth.workload4(dims)
    ws = cp.oracle_weights(wl["layers"], wdtype)
    adt = "bf16" if wdtype == "bf16" else "e4m3"
    scales = _oracle_scales(wl, dims) if adt == "e4m3" else None
    want, sens, bar = _oracle_and_bar(wl, ws, scales, adt)
    kp, vp = _prefixes(wl)
    packed = chain.PackedLayers(wl["layers"], dims, frt.DTYPES[wdtype])
    cd = _run(chain, dims, packed, wl, scales, use_graph=True, keep_intermediates=True)
    d = cp.gpu_dumps(frt, cd, dims, frt.DTYPES[wdtype])
    worst = cp.teacher_forced_check(d, wl["x0"], wl["mod"], kp, vp, ws, scales, dims, adt,
                                    wdtype=wdtype)
    cd.close()
    cpf = _run(chain, dims, packed, wl, scales, use_graph=True, prefetch_next=True)
    got = cpf.read("x_out").reshape(M, -1)
    cpf.close()
    err = rel_l2(got, want)
    log(f"chain {wdtype} M={M} prefix={prefix}: teacher-forced worst {worst}; end to end rel L2 {err:.3e}, "
        f"oracle sensitivity {sens:.3e}")
    record(f"chain 2x2 {wdtype} M={M} prefix={prefix}", _figs(worst, err, sens))
    assert err <= bar
    assert np.array_equal(d["x_out"], got), "production (fused, read-ahead) vs debug chain"


@pytest.mark.parametrize("wdtype", ["bf16", "e4m3"])
def test_chain_wide_hidden(F, wdtype):
    """A wider model than the pages' action decoder: hidden 2048, 16 query heads over the
    one KV head, MLP 4096, M=50, 200 cached keys.  Every GEMM gets other tile shapes (the
    fused merge + O projection 4 column tiles per wave, the down projection's operand 4096
    wide over 2048 columns), checked teacher-forced and end to end as the 1024-wide chain."""
    frt, chain = F
    dims = synth.chain_dims(layers=2, steps=2, M=50, hidden=2048, n_heads=16, prefix=200, mlp=4096)
    wl = synth.workload4(dims)
    ws = cp.oracle_weights(wl["layers"], wdtype)
    adt = "bf16" if wdtype == "bf16" else "e4m3"
    scales = _oracle_scales(wl, dims) if adt == "e4m3" else None
    want, sens, bar = _oracle_and_bar(wl, ws, scales, adt)
    kp, vp = _prefixes(wl)
    packed = chain.PackedLayers(wl["layers"], dims, frt.DTYPES[wdtype])
    cd = _run(chain, dims, packed, wl, scales, use_graph=True, keep_intermediates=True)
    d = cp.gpu_dumps(frt, cd, dims, frt.DTYPES[wdtype])
    worst = cp.teacher_forced_check(d, wl["x0"], wl["mod"], kp, vp, ws, scales, dims, adt,
                                    wdtype=wdtype)
    cd.close()
    cpf = _run(chain, dims, packed, wl, scales, use_graph=True, prefetch_next=True)
    got = cpf.read("x_out").reshape(50, -1)
    cpf.close()
    err = rel_l2(got, want)
    log(f"chain {wdtype} hidden 2048, 16 heads: teacher-forced worst {worst}; end to end rel L2 {err:.3e}, "
        f"oracle sensitivity {sens:.3e}")
    record(f"chain 2x2 {wdtype} M=50 hidden=2048 heads=16", _figs(worst, err, sens))
    assert err <= bar
    assert np.array_equal(d["x_out"], got), "production (fused, read-ahead) vs debug chain"


_FULL = {}


def _full_setup(M, scales_needed):
    """Full-size decision inputs (cached per M) and, when asked for, the oracle's static
    scales (one calibration run per M, shared by the e4m3 and MXFP4 decisions)."""
    if M not in _FULL:
        dims = synth.chain_dims(layers=18, steps=10, M=M)
        _FULL[M] = dict(dims=dims, wl=synth.workload4(dims), scales=None)
    e = _FULL[M]
    if scales_needed and e["scales"] is None:
        t = time.time()
        e["scales"] = _oracle_scales(e["wl"], e["dims"])
        log(f"full decision M={M}: oracle calibration {time.time() - t:.1f} s")
    return e["dims"], e["wl"], e["scales"]


@pytest.mark.parametrize("wdtype,M", [("bf16", 50), ("e4m3", 50), ("mxfp4", 50),
                                      ("bf16", 10), ("e4m3", 10), ("mxfp4", 10)])
def test_full_decision_parity(F, wdtype, M):
    """The benchmark's workload, 18 layers x 10 flow steps, in bf16, e4m3 and MXFP4 weights
    (e4m3 activations with the oracle's calibrated static scales).  The production chain
    (graph replay, weight read-ahead, attention merge fused into the O projection) runs
    in the benchmark's launch configuration and must equal the debug chain bit for bit;
    the debug chain is teacher-forced at every layer of the first and the last flow step;
    the output is compared end to end with the oracle's 180-layer chain (2x sensitivity,
    two noise draws)."""
    frt, chain = F
    adt = "bf16" if wdtype == "bf16" else "e4m3"
    dims, wl, scales = _full_setup(M, adt == "e4m3")
    scales = scales if adt == "e4m3" else None
    ws = cp.oracle_weights(wl["layers"], wdtype)
    t = time.time()
    want, sens, bar = _oracle_and_bar(wl, ws, scales, adt, seeds=(95, 96))
    log(f"full decision {wdtype} M={M}: oracle + sensitivity {time.time() - t:.1f} s")
    packed = chain.PackedLayers(wl["layers"], dims, frt.DTYPES[wdtype])
    ch = _run(chain, dims, packed, wl, scales, use_graph=True, prefetch_next=True)
    got = ch.read("x_out").reshape(M, -1)
    assert ch.kernel_count() == 7 * 18 * 10 + 1
    ch.close()
    err = rel_l2(got, want)
    log(f"full decision {wdtype} M={M}: end to end rel L2 {err:.3e}, oracle sensitivity {sens:.3e}, bar {bar:.3e}")
    cd = _run(chain, dims, packed, wl, scales, use_graph=True, keep_intermediates=True)
    d = cp.gpu_dumps(frt, cd, dims, frt.DTYPES[wdtype])
    cd.close()
    del packed
    torch.cuda.empty_cache()
    assert np.array_equal(d["x_out"], got), "production vs debug chain"
    kp, vp = _prefixes(wl)
    t = time.time()
    worst = cp.teacher_forced_check(d, wl["x0"], wl["mod"], kp, vp, ws, scales, dims, adt, steps=[0, 9],
                                    wdtype=wdtype)
    log(f"full decision {wdtype} M={M}: teacher-forced steps 0 and 9 pass ({time.time() - t:.1f} s), worst {worst}")
    record(f"decision 18x10 {wdtype} M={M}", _figs(worst, err, sens))
    assert err <= bar


def test_weight_read_ahead_leaves_results_bit_identical(F):
    """Reading the down weights ahead (prefetch_next) only reads; outputs must not change."""
    frt, chain = F
    dims = synth.chain_dims(layers=3, steps=2, M=50)
    wl = synth.workload4(dims)
    packed = chain.PackedLayers(wl["layers"], dims, frt.BF16)
    outs, counts = [], []
    for pf in (False, True):
        ch = chain.Chain(dims, packed, use_graph=True, prefetch_next=pf)
        chain.load_workload(ch, wl)
        ch.run()
        ch.run()
        torch.cuda.synchronize()
        outs.append(ch.read("x_out"))
        counts.append(ch.kernel_count())
        ch.close()
    assert np.array_equal(outs[0], outs[1])
    assert counts[0] == counts[1]  # extra workgroups inside existing kernels, no new launches


def test_chain_calibration_matches_oracle(F):
    """GPU calibration (the bf16 chain, max |GEMM input| per site over every step, before
    each input's bf16 rounding) against the oracle's (float64, un-rounded activations,
    same bf16 master weights).  The GPU runs the only chain it has, whose upstream inputs
    are bf16-rounded, so a site's maximum may move by about the bf16 step per upstream
    rounding; the parity tests pass the oracle's scales to both sides."""
    frt, chain = F
    dims = synth.chain_dims(layers=2, steps=3, M=50)
    wl = synth.workload4(dims, input_seed=synth.CAL_SEED)
    packed = chain.PackedLayers(wl["layers"], dims, frt.BF16)
    ch = chain.Chain(dims, packed, use_graph=False)
    chain.load_workload(ch, wl)
    got = ch.calibrate().cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    x_cal = ch.read("x_out").reshape(dims["M"], -1)
    ch.close()
    kp, vp = _prefixes(wl)
    want = ref.calibrate(wl["x0"], cp.oracle_weights(wl["layers"], "bf16"), kp, vp, wl["mod"], dims, 1e-6)
    rel = np.abs(got - want) / want
    log(f"calibration scales rel diff: max {rel.max():.2e}, per site {rel.round(5).tolist()}")
    record("GPU calibration vs oracle (max rel diff of the scales)", f"{rel.max():.2e}")
    assert rel.max() <= 0.02
    assert np.all(np.isfinite(x_cal))
