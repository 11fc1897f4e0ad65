"""Teacher-forced, per-(flow step, layer) parity of the action-decoder chain.

Test infrastructure: it calls the oracle only.  A chain built with debug buffers leaves,
for every (step k, layer l), each kernel's inputs and outputs in the arena.  Each kernel
of each layer-step is then checked against the oracle's step computed from the *GPU's own
inputs to that kernel* (teacher forcing), at the per-kernel bars:

  producer (attention sublayer)  h_attn elementwise within 2^-20 of its summands' size;
                                 QKV operand codes within the tie band
  QKV GEMM + split               Q, own K, own V bf16 codes within the tie band
  attention                      O-projection operand codes within the tie band
  O projection                   fp32 partials, relative L2 <= 1e-5 where the products are
                                 exact (bf16; e4m3 at M <= 16), else 1e-4
  producer (MLP sublayer)        h_mlp as above; gate|up operand codes within the tie band
  gate|up GEMM + SiLU gate       down-projection operand codes within the tie band
  down projection                fp32 partials as for the O projection
  final producer                 x_out as for h_attn

Because every check starts from what the GPU actually read, a wiring mistake at any one
layer-step (a wrong layer's weights, scales, cache or modulation row, a stale buffer)
shows up at that layer-step at kernel tolerance instead of hiding inside the chain's
amplification of rounding differences.  ``oracle_dumps`` produces the same record from the
oracle alone, optionally with a planted wiring mistake, so the CPU tests can show that
the check accepts the oracle and rejects each planted mistake.

Pages: observation-age notes "思考探索：具身推理加速，先看动作执行时观测有多旧", section
"静态量化改变了两次矩阵乘之间的工作" (18 layers x 10 flow steps = 180 passes, each with
FP8 conversion and scale recovery; the consumer prepares the next layer's input with the
next layer's conditioning); section "小 M GEMM 要看并行度，也要看归约代价" (FP32 partials
reduced by the consumer).
"""
import numpy as np

from oracle import codec, ref
from tests.helpers import check_codes, e4m3_products_exact, partial_bar, rel_l2, silu_gate_mag

SITE_QKV, SITE_O, SITE_UP, SITE_DOWN = 0, 1, 2, 3
SCALE, SHIFT, GATE = 0, 1, 2
RES_ULPS = 2.0 ** -20          # residual-stream bound, relative to the size of its summands





def _splits_from_bytes(total, SL, one):
    for s in (1, 2, 4, 8, 16):
        if SL * ((s * one + 255) // 256 * 256) == total:
            return s
    raise ValueError("cannot infer the split count from the debug buffer size")


def gpu_dumps(frt, cg, dims, wdtype):
    """Read a debug chain's per-(step, layer) buffers into logical arrays (numpy)."""
    S, L, M, H = dims["steps"], dims["layers"], dims["M"], dims["hidden"]
    nh, hd, F = dims["n_heads"], dims["head_dim"], dims["mlp"]
    nq = nh * hd
    adt = frt.act_dtype(wdtype)
    Mp = 16 * ((M + 15) // 16)
    SL = S * L
    a256 = lambda b: (b + 255) // 256 * 256  # noqa: E731

    def operands(name, K):
        raw = cg.read(name)
        ob = frt.frt_operand_bytes(adt, M, K)
        step = a256(ob)
        out = np.stack([frt.frt_operand_unpack_host(raw[i * step:i * step + ob], adt, Mp, K)
                        for i in range(SL)])
        assert np.all(out[:, M:] == 0), f"{name}: padding rows must hold zero codes"
        return out[:, :M].reshape((S, L, M, K))

    def rows16(name, width):
        raw = cg.read(name).view(np.uint16)
        step = a256(M * width * 2) // 2
        return np.stack([raw[i * step:i * step + M * width] for i in range(SL)]).reshape(S, L, M, width)

    def partials(name):
        raw = cg.read(name)
        one = M * H * 4
        s = _splits_from_bytes(raw.size * 4, SL, one)
        step = a256(s * one) // 4
        return np.stack([raw[i * step:i * step + s * M * H] for i in range(SL)]).reshape(S, L, s, M, H)

    return dict(
        h_attn=cg.read("dbg_h_attn").reshape(S, L, M, H),
        h_mlp=cg.read("dbg_h_mlp").reshape(S, L, M, H),
        a_qkv=operands("dbg_a_qkv", H), a_o=operands("dbg_a_o", nq),
        a_up=operands("dbg_a_up", H), a_down=operands("dbg_a_down", F),
        q=rows16("dbg_q", nq), k_own=rows16("dbg_k_own", hd), v_own=rows16("dbg_v_own", hd),
        p_o=partials("dbg_p_o"), p_down=partials("dbg_p_down"),
        x_out=cg.read("x_out").reshape(M, H))


def _scale(scales, adt, l, site):
    return float(scales[l][site]) if adt == "e4m3" else 1.0


def _gemm_mag(a_dec, w_dec, s_a, s_w):
    mag = (np.abs(a_dec) @ np.abs(w_dec)) * s_a
    return mag * np.asarray(s_w)[None, :] if s_w is not None else mag


def _check_residual(got, want, r, gate, xmag, label):
    """Elementwise: |GPU - oracle| <= 2^-20 * (|r| + |gate| * xmag), the float32 error of
    h = r + gate * x; xmag = sum_j |P_j| * scales, the size of the summands of x."""
    mag = np.abs(r) + (0.0 if xmag is None else xmag * (1.0 if gate is None else np.abs(gate)[None, :]))
    err = np.abs(np.asarray(got, np.float64) - want)
    bad = err > RES_ULPS * mag + 1e-30
    if bad.any():
        i = np.flatnonzero(bad.ravel())[0]
        raise AssertionError(f"{label}: {int(bad.sum())} of {bad.size} residual values off; first at {i}: "
                             f"gpu {got.ravel()[i]!r} oracle {want.ravel()[i]!r} (rel L2 {rel_l2(got, want):.2e})")


def teacher_forced_check(dumps, x0, mod, kp, vp, ws, scales, dims, adt, steps=None, eps=1e-6, log=None,
                         wdtype=None):
    """Check every kernel of every listed flow step against the oracle on the GPU's own
    inputs.  ws: per-layer oracle weights (decoded values; colscales 's<name>' for e4m3
    weights); scales: [L][4] static activation scales (e4m3 activations) or None;
    wdtype: the weight format ("bf16", "e4m3" or "mxfp4"; default: that of adt).
    Raises AssertionError naming the first (step, layer, kernel) that fails; returns a
    dict of the worst figure per check."""
    S, L, M, H = dims["steps"], dims["layers"], dims["M"], dims["hidden"]
    nh, hd = dims["n_heads"], dims["head_dim"]
    nq = nh * hd
    steps = range(S) if steps is None else steps
    wdtype = wdtype or adt
    exact = wdtype == "bf16" or (wdtype == "e4m3" and e4m3_products_exact(M))
    qkv_frac = 0.01 if exact else 0.05   # bf16 roundings of fp8-MFMA outputs (its internal rounding)
    pbar = partial_bar(wdtype, M)
    worst = dict(h=0.0, p_o=0.0, p_down=0.0, code_frac=0.0)
    dec = lambda c: codec.decode(c, adt)  # noqa: E731

    def codes(got, v, mag, label, dtype=adt, max_frac=0.01):
        n, tot = check_codes(got, v, mag, dtype, max_frac=max_frac, label=label)
        worst["code_frac"] = max(worst["code_frac"], n / tot)

    def prev_of(k, l):
        if l > 0:
            return k, l - 1
        return (k - 1, L - 1) if k > 0 else None

    def producer(k, l, r, parts, lp, gate, sub, site, label):
        x_scale = x_cs = None
        if parts is not None:
            x_scale = _scale(scales, adt, lp, SITE_DOWN if sub == 0 else SITE_O)
            x_cs = ws[lp].get("sdown" if sub == 0 else "so")
        o = ref.residual_norm_quant(r, parts, x_cs, 1.0 if x_scale is None else x_scale, gate,
                                    None if mod is None else mod[k, l, sub, SCALE],
                                    None if mod is None else mod[k, l, sub, SHIFT], eps, adt,
                                    _scale(scales, adt, l, site))
        xmag = None if parts is None else ref.reduce_partials(np.abs(parts), x_scale, x_cs)
        return o, xmag

    for k in steps:
        for l in range(L):
            tag = f"step {k} layer {l}"
            w = ws[l]
            pv = prev_of(k, l)
            # 1. producer: previous layer's down partials + gated residual + AdaRMSNorm
            if pv is None:
                r, parts, gate, lp = np.asarray(x0, np.float64), None, None, None
            else:
                kp_, lp = pv
                r, parts, gate = dumps["h_mlp"][kp_, lp], dumps["p_down"][kp_, lp], mod[kp_, lp, 1, GATE]
            o1, xm = producer(k, l, r, parts, lp, gate, 0, SITE_QKV, tag)
            _check_residual(dumps["h_attn"][k, l], o1["h"], r, gate, xm, f"{tag}: h entering attention")
            worst["h"] = max(worst["h"], rel_l2(dumps["h_attn"][k, l], o1["h"]))
            codes(dumps["a_qkv"][k, l], o1["v"], o1["mag"], f"{tag}: QKV operand")
            # 2. QKV GEMM -> bf16 Q, own K, own V (from the GPU's operand codes)
            s_a = _scale(scales, adt, l, SITE_QKV)
            a = dec(dumps["a_qkv"][k, l])
            c = ref.reduce_partials(ref.gemm_splitk(a, w["qkv"], 1), s_a, w.get("sqkv"))
            mg = _gemm_mag(a, w["qkv"], s_a, w.get("sqkv"))
            codes(dumps["q"][k, l], c[:, :nq], mg[:, :nq], f"{tag}: Q", "bf16", qkv_frac)
            codes(dumps["k_own"][k, l], c[:, nq:nq + hd], mg[:, nq:nq + hd], f"{tag}: own K", "bf16", qkv_frac)
            codes(dumps["v_own"][k, l], c[:, nq + hd:], mg[:, nq + hd:], f"{tag}: own V", "bf16", qkv_frac)
            # 3. attention over [prefix; own rows] (the GPU's Q, K, V) -> O operand codes
            kall = np.concatenate([kp[l], codec.bf16_decode(dumps["k_own"][k, l])])
            vall = np.concatenate([vp[l], codec.bf16_decode(dumps["v_own"][k, l])])
            o, mag = ref.attention_prefix(codec.bf16_decode(dumps["q"][k, l]), kall, vall, nh, hd)
            s_o = _scale(scales, adt, l, SITE_O)
            v, _, _ = ref.quantise(o, adt, s_o)
            codes(dumps["a_o"][k, l], v, mag / s_o, f"{tag}: O-projection operand")
            # 4. O projection partials
            p_o = dumps["p_o"][k, l]
            want = ref.gemm_splitk(dec(dumps["a_o"][k, l]), w["o"], p_o.shape[0])
            e = rel_l2(p_o, want)
            worst["p_o"] = max(worst["p_o"], e)
            assert e <= pbar, f"{tag}: O-projection partials rel L2 {e:.2e} > {pbar:g}"
            # 5. producer: attention output + gated residual + AdaRMSNorm (MLP sublayer)
            r2, g2 = dumps["h_attn"][k, l], mod[k, l, 0, GATE]
            o2, xm2 = producer(k, l, r2, p_o, l, g2, 1, SITE_UP, tag)
            _check_residual(dumps["h_mlp"][k, l], o2["h"], r2, g2, xm2, f"{tag}: h entering the MLP")
            worst["h"] = max(worst["h"], rel_l2(dumps["h_mlp"][k, l], o2["h"]))
            codes(dumps["a_up"][k, l], o2["v"], o2["mag"], f"{tag}: gate|up operand")
            # 6. gate|up GEMM + SiLU(gate) * up -> down operand codes
            s_u, s_d = _scale(scales, adt, l, SITE_UP), _scale(scales, adt, l, SITE_DOWN)
            a = dec(dumps["a_up"][k, l])
            c_up = ref.reduce_partials(ref.gemm_splitk(a, w["up"], 1), s_u, w.get("sup"))
            z = ref.silu_gate_quant(c_up, adt, s_d)
            codes(dumps["a_down"][k, l], z["v"], silu_gate_mag(c_up, a, w["up"], s_u, w.get("sup"), adt, s_d),
                  f"{tag}: down operand")
            # 7. down projection partials
            p_d = dumps["p_down"][k, l]
            want = ref.gemm_splitk(dec(dumps["a_down"][k, l]), w["down"], p_d.shape[0])
            e = rel_l2(p_d, want)
            worst["p_down"] = max(worst["p_down"], e)
            assert e <= pbar, f"{tag}: down-projection partials rel L2 {e:.2e} > {pbar:g}"
        if log:
            log(f"teacher-forced step {k}: all {L} layers pass (worst so far {worst})")
    if S - 1 in steps:
        # final producer: last MLP output into x_out
        fin, xm = producer(S - 1, L - 1, dumps["h_mlp"][S - 1, L - 1], dumps["p_down"][S - 1, L - 1], L - 1,
                           mod[S - 1, L - 1, 1, GATE], 0, SITE_QKV, "final")
        _check_residual(dumps["x_out"], fin["h"], dumps["h_mlp"][S - 1, L - 1], mod[S - 1, L - 1, 1, GATE], xm,
                        "final residual x_out")
    return worst


# ------------------------------------------------------------------ the same record from the oracle

PLANTS = ("down_colscale_of_previous_layer", "kv_prefix_of_previous_layer", "modulation_of_previous_step",
          "attention_gate_for_mlp_residual", "stale_down_partials")


def oracle_dumps(x0, mod, kp, vp, ws, scales, dims, adt, s_o=2, s_down=2, eps=1e-6, plant=None):
    """What a correct debug chain leaves in its buffers, computed by the oracle alone,
    with optionally one planted wiring mistake (CPU tests of the check itself)."""
    assert plant is None or plant in PLANTS
    S, L, M, H = dims["steps"], dims["layers"], dims["M"], dims["hidden"]
    nh, hd, F = dims["n_heads"], dims["head_dim"], dims["mlp"]
    nq = nh * hd
    out = {n: [[None] * L for _ in range(S)] for n in
           ("h_attn", "h_mlp", "a_qkv", "a_o", "a_up", "a_down", "q", "k_own", "v_own", "p_o", "p_down")}
    sc = lambda l, site: _scale(scales, adt, l, site)  # noqa: E731
    h, parts, gate, lp, lpp = np.asarray(x0, np.float64), None, None, None, None
    for k in range(S):
        for l in range(L):
            m0 = mod[k - 1 if (plant == "modulation_of_previous_step" and k > 0) else k, l]
            cs = None
            if parts is not None:
                cs = ws[lp].get("sdown")
                if plant == "down_colscale_of_previous_layer" and lp >= 1:
                    cs = ws[lp - 1].get("sdown")
            x_parts = parts
            if plant == "stale_down_partials" and lpp is not None and (k, l) == (S - 1, L - 1):
                x_parts = lpp
            o1 = ref.residual_norm_quant(h, x_parts, cs, 1.0 if parts is None else sc(lp, SITE_DOWN), gate,
                                         m0[0, SCALE], m0[0, SHIFT], eps, adt, sc(l, SITE_QKV))
            out["h_attn"][k][l], out["a_qkv"][k][l] = o1["h"], o1["codes"]
            c = ref.reduce_partials(ref.gemm_splitk(o1["deq"], ws[l]["qkv"], 1), sc(l, SITE_QKV), ws[l].get("sqkv"))
            qkv = codec.bf16_encode(c)
            out["q"][k][l], out["k_own"][k][l], out["v_own"][k][l] = qkv[:, :nq], qkv[:, nq:nq + hd], qkv[:, nq + hd:]
            lk = l - 1 if (plant == "kv_prefix_of_previous_layer" and l >= 1) else l
            att = ref.attention_block(c, kp[lk], vp[lk], nh, hd, adt, sc(l, SITE_O))
            out["a_o"][k][l] = att["codes"]
            p_o = ref.gemm_splitk(att["deq"], ws[l]["o"], s_o)
            out["p_o"][k][l] = p_o
            g_attn = m0[1, GATE] if plant == "attention_gate_for_mlp_residual" else m0[0, GATE]
            o2 = ref.residual_norm_quant(o1["h"], p_o, ws[l].get("so"), sc(l, SITE_O), g_attn,
                                         m0[1, SCALE], m0[1, SHIFT], eps, adt, sc(l, SITE_UP))
            out["h_mlp"][k][l], out["a_up"][k][l] = o2["h"], o2["codes"]
            c_up = ref.reduce_partials(ref.gemm_splitk(o2["deq"], ws[l]["up"], 1), sc(l, SITE_UP), ws[l].get("sup"))
            z = ref.silu_gate_quant(c_up, adt, sc(l, SITE_DOWN))
            out["a_down"][k][l] = z["codes"]
            lpp = parts
            parts = ref.gemm_splitk(z["deq"], ws[l]["down"], s_down)
            out["p_down"][k][l] = parts
            h, gate, lp = o2["h"], m0[1, GATE], l
    cs = ws[lp].get("sdown")
    if plant == "down_colscale_of_previous_layer" and lp >= 1:
        cs = ws[lp - 1].get("sdown")
    fin = ref.residual_norm_quant(h, parts, cs, sc(lp, SITE_DOWN), gate, eps=eps, out_dtype=adt)
    d = {n: np.array(v) for n, v in out.items()}
    d["x_out"] = fin["h"]
    return d


def oracle_weights(layers, wdtype):
    """Oracle-side weights of a layer stack from its bf16 master weights: decoded values of
    the packed format, plus per-column scales ('s<name>') for e4m3 weights."""
    ws = []
    for lw in layers:
        d = {}
        for name in ("qkv", "o", "up", "down"):
            if wdtype == "mxfp4":
                d[name] = ref.pack_weight_mxfp4(codec.bf16_decode(lw[name]))[2]
                continue
            codes, s_w, _ = ref.pack_weight_values(codec.bf16_decode(lw[name]), None, wdtype)
            d[name] = codec.decode(codes, wdtype)
            if s_w is not None:
                d["s" + name] = s_w
        ws.append(d)
    return ws


def sensitivity(run, want, noise, seeds=(95, 96, 97)):
    """How far the oracle chain itself moves when every GEMM input is perturbed by relative
    noise of the given size before rounding: the largest relative L2 change over a few
    noise draws (the count of rounding flips such noise causes is itself random)."""
    out = 0.0
    for s in seeds:
        g = np.random.default_rng(s)
        out = max(out, rel_l2(run(lambda v: v * (1.0 + noise * g.standard_normal(v.shape))), want))
    return out
