"""Persistent chain state on MI355X: the execution-state capsule (snapshot, restore, fork)
and selective refresh of the state between decisions (abstract page: execution-state
capsule; observation-age notes: state reuse keeps outputs bit-identical).

Replay uses fixed addresses, so the state a decision runs on lives in named buffers that
persist across runs.  These tests check, bit for bit, that
- restoring a snapshot into the same chain, or forking it into a second chain, reproduces
  the decision taken from that state;
- re-uploading only the part of the state that changed (a new observation in "x_in", new
  prefix keys/values of one layer) gives exactly what a freshly built chain computes from
  the full new state -- nothing stale from the previous decision leaks into the next.
Each restored, forked or refreshed decision is also held to the oracle chain run on the
inputs that decision stands for (end to end, twice the oracle's own sensitivity to
2^-22 relative noise on its GEMM inputs, as for the chain's own parity tests).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import codec, ref
from tests import chain_parity as cp
from tests.helpers import rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def F():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X GPU")
    from gemm_chains_amd import chain, frt
    frt.lib()
    dims = synth.chain_dims(layers=3, steps=2, M=50)
    wl = synth.workload4(dims)
    packed = chain.PackedLayers(wl["layers"], dims, frt.BF16)
    return frt, chain, dims, wl, packed


def _decide(ch):
    ch.run()
    torch.cuda.synchronize()
    return ch.read("x_out")


def _oracle_check(got, wl, label):
    """End to end against the oracle chain on the inputs `wl` (x0, layers, mod)."""
    dims = wl["dims"]
    ws = cp.oracle_weights(wl["layers"], "bf16")
    kp = [codec.bf16_decode(l["k_prefix"]) for l in wl["layers"]]
    vp = [codec.bf16_decode(l["v_prefix"]) for l in wl["layers"]]

    def run(perturb=None):
        return ref.chain(wl["x0"], ws, np.ones((dims["layers"], 4)), kp, vp, wl["mod"], dims, "bf16", 1e-6,
                         perturb=perturb)
    want = run()
    sens = cp.sensitivity(run, want, 2.0 ** -22)
    err = rel_l2(np.asarray(got).reshape(want.shape), want)
    print(f"{label}: rel L2 vs oracle {err:.3e} (oracle sensitivity {sens:.3e})", flush=True)
    assert err <= 2.0 * max(sens, 1e-7), label


def test_capsule_snapshot_restore_and_fork(F):
    frt, chain, dims, wl, packed = F
    a = chain.Chain(dims, packed, use_graph=True)
    chain.load_workload(a, wl)
    out1 = _decide(a)
    cap = a.snapshot()
    torch.cuda.synchronize()
    assert cap.numel() == a.state_bytes() > 256
    n = a.state_bytes() - 256                      # the state region; a 256-byte trailer follows
    state = a.arena[:n].clone()
    assert torch.equal(cap[:n], state)
    # a different decision state
    x_new, mod_new = synth.chain_inputs(dims, seed=3)
    a.write("x_in", x_new)
    a.write("mod", mod_new)
    out2 = _decide(a)
    assert not np.array_equal(out1, out2)
    # restore: the state region is the capsule again, and the decision is reproduced
    a.restore(cap)
    torch.cuda.synchronize()
    assert torch.equal(a.arena[:n], cap[:n])
    out3 = _decide(a)
    assert np.array_equal(out1, out3)
    _oracle_check(out3, wl, "restored decision")
    _oracle_check(out2, dict(wl, x0=x_new, mod=mod_new), "decision on the second state")
    # fork into a second chain with its own arena
    b = chain.Chain(dims, packed, use_graph=True)
    b.restore(cap)
    out4 = _decide(b)
    assert np.array_equal(out1, out4)
    _oracle_check(out4, wl, "forked decision")
    assert torch.equal(state[:a.view("x_in").numel() * 4], cap[:a.view("x_in").numel() * 4])
    # the capsule must not alias the arena, and must be exactly state_bytes long
    with pytest.raises(frt.FrtError) as e:
        frt.frt_layer_chain_snapshot(a.handle, a.arena, a.state_bytes())
    assert e.value.status == frt.E_ALIAS
    for n in (a.state_bytes() - 16, a.state_bytes() + 16):
        with pytest.raises(frt.FrtError) as e:
            frt.frt_layer_chain_restore(a.handle, cap, n)
        assert e.value.status == frt.E_WORKSPACE
    a.close()
    b.close()


def test_capsule_restores_only_into_a_chain_of_its_shape(F):
    """A capsule carries a token of its chain's shape fields and state layout; restoring it
    into a chain of another shape (other M, other layer count, other prefix length) or
    from a damaged trailer is refused with FRT_E_STATE and leaves that chain's state as it
    was."""
    frt, chain, dims, wl, packed = F
    a = chain.Chain(dims, packed, use_graph=True)
    chain.load_workload(a, wl)
    out_a = _decide(a)
    cap = a.snapshot()
    torch.cuda.synchronize()
    others = [dict(dims, M=10), dict(dims, prefix=dims["prefix"] - 32)]
    for od in others:
        ow = synth.workload4(od)
        b = chain.Chain(od, packed, use_graph=True)
        chain.load_workload(b, ow)
        before = _decide(b)
        state_b = b.arena[:b.state_bytes() - 256].clone()
        n = min(b.state_bytes(), cap.numel())
        c2 = torch.zeros(b.state_bytes(), dtype=torch.uint8, device="cuda")
        c2[:n] = cap[:n]
        c2[-256:] = cap[-256:]                     # a's trailer on a capsule of b's size
        with pytest.raises(frt.FrtError) as e:
            b.restore(c2)
        assert e.value.status == frt.E_STATE, od
        torch.cuda.synchronize()
        assert torch.equal(b.arena[:b.state_bytes() - 256], state_b)
        assert np.array_equal(_decide(b), before)
        b.close()
    # fewer layers: the same per-layer sizes, another state layout
    pl = chain.PackedLayers(wl["layers"][:2], dict(dims, layers=2), frt.BF16)
    b = chain.Chain(dict(dims, layers=2), pl, use_graph=True)
    c3 = torch.zeros(b.state_bytes(), dtype=torch.uint8, device="cuda")
    c3[-256:] = cap[-256:]
    with pytest.raises(frt.FrtError) as e:
        b.restore(c3)
    assert e.value.status == frt.E_STATE
    b.close()
    # a damaged trailer is refused by a chain of the right shape too
    bad = cap.clone()
    bad[-256 + 8] ^= 1
    with pytest.raises(frt.FrtError) as e:
        a.restore(bad)
    assert e.value.status == frt.E_STATE
    a.restore(cap)
    assert np.array_equal(_decide(a), out_a)
    a.close()


def test_selective_refresh_matches_a_fresh_chain(F):
    frt, chain, dims, wl, packed = F
    a = chain.Chain(dims, packed, use_graph=True)
    chain.load_workload(a, wl)
    _decide(a)
    # new observation: only x_in changes
    x_new, _ = synth.chain_inputs(dims, seed=2)
    a.write("x_in", x_new)
    got = _decide(a)
    b = chain.Chain(dims, packed, use_graph=True)
    chain.load_workload(b, dict(wl, x0=x_new))
    want = _decide(b)
    assert np.array_equal(got, want)
    _oracle_check(got, dict(wl, x0=x_new), "x_in refresh")
    # new prefix keys/values for layer 1 only (a new VLM context for that layer)
    P, hd, T = dims["prefix"], dims["head_dim"], dims["prefix"] + dims["M"]
    ldv = (T + 31) // 32 * 32
    kp = synth.to_bf16_bits(synth.normal(7, 4, 999, (P, hd)))
    vp = synth.to_bf16_bits(synth.normal(7, 4, 998, (P, hd)))
    for ch in (a, b):
        kc = ch.view("k_cache").view(dims["layers"], T, hd)
        vc = ch.view("v_cache").view(dims["layers"], hd, ldv)
        kc[1, :P].copy_(torch.from_numpy(kp.view(np.int16)).cuda())
        vc[1, :, :P].copy_(torch.from_numpy(np.ascontiguousarray(vp.T).view(np.int16)).cuda())
    got2 = _decide(a)
    layers = [dict(l) for l in wl["layers"]]
    layers[1]["k_prefix"], layers[1]["v_prefix"] = kp, vp
    c = chain.Chain(dims, packed, use_graph=True)
    chain.load_workload(c, dict(wl, x0=x_new, layers=layers))
    want2 = _decide(c)
    assert np.array_equal(got2, want2)
    _oracle_check(got2, dict(wl, x0=x_new, layers=layers), "x_in + one layer's prefix refresh")
    assert np.array_equal(_decide(b), want2)
    a.close()
    b.close()
    c.close()
