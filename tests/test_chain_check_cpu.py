"""The teacher-forced chain check (tests/chain_parity.py) on the CPU: it accepts a correct
chain record and rejects plausible wiring mistakes, each planted in an oracle-computed
record (no GPU involved).

The mistakes are the kind a chain builder can make with one wrong pointer or index: the
down projection of layer l reduced with layer l-1's per-column weight scales, layer l
attending over layer l-1's cached prefix, a flow step using the previous step's
modulation rows, the MLP residual gated with the wrong sublayer's gate, and a producer
reading down-projection partials two layers old.  Each changes the chain's final output
by less than the end-to-end bars that rest on the oracle's own sensitivity (0.1 and more
for e4m3), so only a per-layer-step check can be relied on to see them.
"""
import numpy as np
import pytest

import synth
from oracle import codec, ref
from tests import chain_parity as cp
from tests.helpers import rel_l2


def _setup(dims, wdtype):
    wl = synth.workload4(dims)
    ws = cp.oracle_weights(wl["layers"], wdtype)
    kp = [codec.bf16_decode(l["k_prefix"]) for l in wl["layers"]]
    vp = [codec.bf16_decode(l["v_prefix"]) for l in wl["layers"]]
    adt = "bf16" if wdtype == "bf16" else "e4m3"
    scales = None
    if adt == "e4m3":
        x0c, modc = synth.chain_inputs(dims, synth.CAL_SEED)
        scales = ref.calibrate(x0c, cp.oracle_weights(wl["layers"], "bf16"), kp, vp, modc, dims, 1e-6)
    return wl, ws, kp, vp, scales, adt


SMALL = dict(layers=2, steps=2, M=16, hidden=256, n_heads=2, head_dim=128, prefix=64, mlp=512)


@pytest.mark.parametrize("wdtype", ["bf16", "e4m3", "mxfp4"])
def test_check_accepts_the_oracle_record(wdtype):
    dims = synth.chain_dims(**SMALL)
    wl, ws, kp, vp, scales, adt = _setup(dims, wdtype)
    d = cp.oracle_dumps(wl["x0"], wl["mod"], kp, vp, ws, scales, dims, adt)
    # the decomposed record is the oracle chain itself
    want = ref.chain(wl["x0"], ws, scales if scales is not None else np.ones((dims["layers"], 4)),
                     kp, vp, wl["mod"], dims, adt, 1e-6)
    assert rel_l2(d["x_out"], want) <= 1e-12
    worst = cp.teacher_forced_check(d, wl["x0"], wl["mod"], kp, vp, ws, scales, dims, adt)
    assert worst["code_frac"] == 0.0


@pytest.mark.parametrize("plant", cp.PLANTS)
def test_check_rejects_planted_wiring_mistakes(plant):
    dims = synth.chain_dims(**SMALL)
    wl, ws, kp, vp, scales, adt = _setup(dims, "e4m3")
    d = cp.oracle_dumps(wl["x0"], wl["mod"], kp, vp, ws, scales, dims, adt, plant=plant)
    with pytest.raises(AssertionError):
        cp.teacher_forced_check(d, wl["x0"], wl["mod"], kp, vp, ws, scales, dims, adt)


def test_check_rejects_the_wrong_layer_column_scales_at_full_width():
    """The mistake at the chain's real width (hidden 1024, MLP 4096, 8 heads, 800-token
    prefix, M = 50, e4m3, 2 layers x 2 steps): layer 1's down projection reduced with
    layer 0's per-column weight scales.  End to end it moves the output by about a tenth,
    under the e4m3 sensitivity bar; teacher-forced it fails at the first producer that
    reads layer 1's output."""
    dims = synth.chain_dims(layers=2, steps=2, M=50)
    wl, ws, kp, vp, scales, adt = _setup(dims, "e4m3")
    good = cp.oracle_dumps(wl["x0"], wl["mod"], kp, vp, ws, scales, dims, adt, s_o=8, s_down=4)
    cp.teacher_forced_check(good, wl["x0"], wl["mod"], kp, vp, ws, scales, dims, adt)
    bad = cp.oracle_dumps(wl["x0"], wl["mod"], kp, vp, ws, scales, dims, adt, s_o=8, s_down=4,
                          plant="down_colscale_of_previous_layer")
    moved = rel_l2(bad["x_out"], good["x_out"])
    print(f"planted wrong-layer column scales move the output by rel L2 {moved:.3f}")
    assert 0.01 < moved < 0.5
    with pytest.raises(AssertionError, match="step 1 layer 0: h entering attention"):
        cp.teacher_forced_check(bad, wl["x0"], wl["mod"], kp, vp, ws, scales, dims, adt)
