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
"""
import numpy as np
import pytest
import torch

import synth

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


def test_capsule_snapshot_restore_and_fork(F):
    frt, chain, dims, wl, packed = F
    a = chain.Chain(dims, packed, use_graph=True)
    chain.load_workload(a, wl)
    out1 = _decide(a)
    cap = a.snapshot()
    torch.cuda.synchronize()
    assert cap.numel() == a.state_bytes() > 0
    state = a.arena[:a.state_bytes()].clone()
    # a different decision state
    x_new, mod_new = synth.chain_inputs(dims, seed=3)
    a.write("x_in", x_new)
    a.write("mod", mod_new)
    out2 = _decide(a)
    assert not np.array_equal(out1, out2)
    # restore: the state region is the capsule again, and the decision is reproduced
    a.restore(cap)
    torch.cuda.synchronize()
    assert torch.equal(a.arena[:a.state_bytes()], cap)
    out3 = _decide(a)
    assert np.array_equal(out1, out3)
    # fork into a second chain with its own arena
    b = chain.Chain(dims, packed, use_graph=True)
    b.restore(cap)
    out4 = _decide(b)
    assert np.array_equal(out1, out4)
    assert torch.equal(state[:a.view("x_in").numel() * 4], cap[:a.view("x_in").numel() * 4])
    # the capsule must not alias the arena, and must be large enough
    with pytest.raises(frt.FrtError):
        frt.frt_layer_chain_snapshot(a.handle, a.arena, a.state_bytes())
    with pytest.raises(frt.FrtError):
        frt.frt_layer_chain_restore(a.handle, cap, a.state_bytes() - 16)
    a.close()
    b.close()


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
    assert np.array_equal(_decide(b), want2)
    a.close()
    b.close()
    c.close()
