"""Plain float64 reference of the action-decoder layer chain (CPU, NumPy).

TEST INFRASTRUCTURE ONLY.  Nothing outside ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import this package, and it
imports nothing from the GPU library: it shares no code, table, layout or
constant generator with it.  Every step is written out in the order the pages
state it, with no blocking, fusion or reordering; library primitives used are
``numpy.matmul`` (``@``), ``numpy.exp`` and ``numpy.sqrt``.

Pages cited (by title and section):
  [notes]    "思考探索：具身推理加速，先看动作执行时观测有多旧" (observation-age notes on
             the talk 推理加速的系统方法); sections "CUDA Graph 与图化简分别省掉什么"
             (RMSNorm equation, the W' = diag(gamma) W equation, QKV merge,
             producer-consumer fusion), "静态量化改变了两次矩阵乘之间的工作"
             (static activation scales, FP8 conversion and scale recovery repeated
             per layer and step, gated residual + AdaRMSNorm + FP8 conversion as one
             fused op, next-layer conditioning used to prepare the next input),
             "小 M GEMM 要看并行度，也要看归约代价" (C = AW with small M, the
             split-K sum equation, FP32 partials reduced by the consumer).
  [news]     rebasdaily FlashRT-PAI news summary, section "它优化的是“接力方式”"
             (fused FP8 action-decoder layer; compact hand-off layout).
  [abstract] "FlashRT-PAI: Fast Kernels Are Not Fast Pipelines for Physical AI
             Inference" (fusion of operator boundaries; named buffers retained
             across decisions).

Readings taken where the pages are silent (each is listed again in the design notes):
  R1 AdaRMSNorm: y = xhat * (1 + scale) + shift; no separate gamma.
  R2 gated residual: h = r + gate * x, gate belonging to the sublayer that produced x.
  R3 eps inside the square root, eps = 1e-6.
  R4 static activation scale per GEMM-input site: codes = e4m3(y / s_a).
  R5 per-output-channel weight scale s_w[n] = max_k |W[k, n]| / 448, rounded to fp32;
     a column of zeros gets s_w = 0 and all-zero codes.
  R6 scale recovery after the split-K sum: C = (sum_j P_j) * s_a * s_w[n].
  R7 split-K: s contiguous equal K-chunks; partial j covers rows [j*K/s, (j+1)*K/s) of W.
  R8 gate|up: columns [0, N/2) are the gate, [N/2, N) the up projection.
  R9 attention: keys/values = cached prefix followed by the M own rows, one KV head
     shared by every query head, scale 1/sqrt(head_dim), no mask; Q, own K, own V
     are rounded to bf16 before use (they are stored in that format).
  R10 flow steps compose: the residual stream leaving step k enters step k+1.
  R16 4-bit weights (the pages' 4-bit weight path, on gfx950's microscaling matrix
      cores): OCP MXFP4 -- 32 consecutive k of a column share an E8M0 scale
      2**(floor(log2 max|w|) - 2); elements are FP4 E2M1, round to nearest even,
      saturating at 6; an all-zero block gets scale byte 0.  Activations stay e4m3
      with their static per-site scales; the block scales replace s_w.
"""
import numpy as np

from . import codec


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def f32(a):
    """Round float64 values to the nearest float32 value (library cast, RNE)."""
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


# ----------------------------------------------------------------- norms

def rms_normalise(h, eps):
    """xhat = h / sqrt(mean(h^2) + eps), row-wise ([notes] RMSNorm equation)."""
    h = _f64(h)
    ms = np.mean(h * h, axis=-1, keepdims=True)
    return h / np.sqrt(ms + eps)


def rmsnorm_matmul(x, gamma, w, eps):
    """The plain definition y = (xhat * gamma) W ([notes] RMSNorm equation)."""
    return (rms_normalise(x, eps) * _f64(gamma)[None, :]) @ _f64(w)


def fold_gamma(gamma, w):
    """W' = diag(gamma) W: row k of W scaled by gamma[k] ([notes] the W' equation)."""
    return _f64(gamma)[:, None] * _f64(w)


def gated_residual(r, gate, x):
    """h = r + gate * x (reading R2); gate None means 1, x None means no update."""
    r = _f64(r)
    if x is None:
        return r.copy()
    x = _f64(x)
    if gate is None:
        return r + x
    return r + _f64(gate)[None, :] * x


def ada_modulate(xhat, scale, shift):
    """y = xhat * (1 + scale) + shift (reading R1); None means 0 for either vector."""
    y = _f64(xhat)
    if scale is not None:
        y = y * (1.0 + _f64(scale)[None, :])
    if shift is not None:
        y = y + _f64(shift)[None, :]
    return y


def quantise(v, dtype, act_scale=1.0):
    """Static-scale quantisation of a GEMM input (reading R4).

    Returns (pre-rounding value, codes, decoded values).  For bf16 the scale is 1.
    """
    v = _f64(v)
    if dtype == "e4m3":
        v = v / act_scale
    codes = codec.encode(v, dtype)
    return v, codes, codec.decode(codes, dtype)


def residual_norm_quant(residual, x_parts=None, x_colscale=None, x_scale=1.0, gate=None,
                        ada_scale=None, ada_shift=None, eps=1e-6, out_dtype="bf16",
                        act_scale=1.0):
    """Producer step: [reduce partials, dequant] -> gated residual -> (Ada)RMSNorm -> quantise.

    x_parts: [s][M][K] partial sums of the previous GEMM or None; they are summed in
    ascending j (reading R6/R7) and scaled by x_scale * x_colscale[k].
    Returns a dict with h (new residual stream), xhat, y, v (value that is rounded),
    codes, deq (decoded codes) and mag (size of the summands of y, scaled like v; used
    to size the rounding tie band in comparisons).
    """
    x = None
    if x_parts is not None:
        x = reduce_partials(x_parts, x_scale, x_colscale)
    h = gated_residual(residual, gate, x)
    xhat = rms_normalise(h, eps)
    y = ada_modulate(xhat, ada_scale, ada_shift)
    # size of the summands of y: (|r| + |gate * x|) / rms scaled by |1 + scale|, plus |shift|
    hmag = np.abs(gated_residual(np.abs(_f64(residual)), None if gate is None else np.abs(_f64(gate)),
                                 None if x is None else np.abs(x)))
    inv_rms = 1.0 / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)
    mag = np.abs(ada_modulate(hmag * inv_rms, ada_scale, None))
    if ada_shift is not None:
        mag = mag + np.abs(_f64(ada_shift))[None, :]
    v, codes, deq = quantise(y, out_dtype, act_scale)
    if out_dtype == "e4m3":
        mag = mag / act_scale
    return dict(h=h, xhat=xhat, y=y, v=v, codes=codes, deq=deq, mag=mag)


# ----------------------------------------------------------------- weights

def pack_weight_values(w_bf16_values, gamma, dtype):
    """Offline weight preparation.

    bf16: codes of W' = diag(gamma) W rounded to bf16 (gamma None: W itself).
    e4m3: W' as above in float64, s_w[n] = fp32(max_k |W'[k,n]| / 448) (reading R5),
          codes = e4m3(W' / s_w[n]).
    Returns (codes [K][N], colscale [N] or None, pre-rounding values [K][N]).
    """
    w = _f64(w_bf16_values)
    if gamma is not None:
        w = fold_gamma(gamma, w)
    if dtype == "bf16":
        return codec.bf16_encode(w), None, w
    amax = np.max(np.abs(w), axis=0)
    s_w = f32(amax / codec.E4M3_MAX)
    safe = np.where(s_w > 0, s_w, 1.0)
    v = np.where(s_w[None, :] > 0, w / safe[None, :], 0.0)
    return codec.e4m3_encode(v), s_w, v


def pack_weight_mxfp4(w_bf16_values, gamma=None):
    """Offline weight preparation for 4-bit weights (OCP MXFP4, reading R16).

    W' = diag(gamma) W (float64), then blocks of 32 consecutive k of each column share an
    E8M0 scale and the elements are FP4 E2M1 codes (codec.mxfp4_encode).  The GEMM uses
    the decoded values W'' = code * 2**(scale - 127); no per-column scale remains.
    Returns (codes [K][N], scale bytes [K/32][N], decoded values [K][N]).
    """
    w = _f64(w_bf16_values)
    if gamma is not None:
        w = fold_gamma(gamma, w)
    codes, sb, _ = codec.mxfp4_encode(w)
    return codes, sb, codec.mxfp4_decode(codes, sb)


# ----------------------------------------------------------------- GEMM

def gemm_splitk(a, w, splits):
    """P_j = A[:, K_j] W[K_j, :] for s contiguous equal K-chunks ([notes] split-K equation)."""
    a = _f64(a)
    w = _f64(w)
    K = a.shape[1]
    if K % splits:
        raise ValueError("K must divide into equal chunks")
    kc = K // splits
    return np.stack([a[:, j * kc:(j + 1) * kc] @ w[j * kc:(j + 1) * kc, :]
                     for j in range(splits)])


def reduce_partials(parts, act_scale=1.0, colscale=None):
    """C = (sum over j ascending of P_j) * act_scale * colscale[n] (reading R6)."""
    parts = _f64(parts)
    c = parts[0].copy()
    for j in range(1, parts.shape[0]):
        c = c + parts[j]
    c = c * act_scale
    if colscale is not None:
        c = c * _f64(colscale)[None, :]
    return c


def silu(g):
    """SiLU(g) = g / (1 + exp(-g))."""
    g = _f64(g)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def silu_gate(c):
    """z = SiLU(gate) * up with C = [gate | up] along columns (reading R8)."""
    c = _f64(c)
    n2 = c.shape[1] // 2
    return silu(c[:, :n2]) * c[:, n2:]


def silu_gate_quant(c, dtype, act_scale=1.0):
    """Consumer epilogue (ii): SiLU-gate then quantise for the down projection."""
    c = _f64(c)
    n2 = c.shape[1] // 2
    z = silu_gate(c)
    mag = np.abs(silu(c[:, :n2])) * np.abs(c[:, n2:])
    v, codes, deq = quantise(z, dtype, act_scale)
    if dtype == "e4m3":
        mag = mag / act_scale
    return dict(z=z, v=v, codes=codes, deq=deq, mag=mag)


# ----------------------------------------------------------------- attention

def attention_prefix(q, k_all, v_all, n_heads, head_dim):
    """softmax(q_h K^T / sqrt(d)) V for each query head h, one KV head shared (reading R9).

    q: [M][n_heads*head_dim]; k_all, v_all: [T][head_dim].
    Returns (O [M][n_heads*head_dim], mag) where mag[m, h*d+e] = sum_t p_t |V[t,e]|,
    the size of the summands of each output.
    """
    q = _f64(q)
    k_all = _f64(k_all)
    v_all = _f64(v_all)
    out = np.empty_like(q)
    mag = np.empty_like(q)
    for h in range(n_heads):
        qh = q[:, h * head_dim:(h + 1) * head_dim]
        s = (qh @ k_all.T) / np.sqrt(head_dim)
        s = s - np.max(s, axis=1, keepdims=True)
        p = np.exp(s)
        p = p / np.sum(p, axis=1, keepdims=True)
        out[:, h * head_dim:(h + 1) * head_dim] = p @ v_all
        mag[:, h * head_dim:(h + 1) * head_dim] = p @ np.abs(v_all)
    return out, mag


def qkv_split_bf16(c_qkv, n_heads, head_dim):
    """Split the fused QKV output [M][(n_heads+2)*head_dim] into Q, own K, own V, rounded to bf16."""
    c = _f64(c_qkv)
    nq = n_heads * head_dim
    r = codec.bf16_round(c)
    return r[:, :nq], r[:, nq:nq + head_dim], r[:, nq + head_dim:nq + 2 * head_dim]


def attention_block(c_qkv, k_prefix, v_prefix, n_heads, head_dim, out_dtype, act_scale=1.0):
    """QKV output -> bf16 Q/K/V -> attention over [prefix; own] -> quantised O-proj operand."""
    qb, kb, vb = qkv_split_bf16(c_qkv, n_heads, head_dim)
    k_all = np.concatenate([_f64(k_prefix), kb], axis=0)
    v_all = np.concatenate([_f64(v_prefix), vb], axis=0)
    o, mag = attention_prefix(qb, k_all, v_all, n_heads, head_dim)
    v, codes, deq = quantise(o, out_dtype, act_scale)
    if out_dtype == "e4m3":
        mag = mag / act_scale
    return dict(q=qb, k=kb, v_own=vb, o=o, v=v, codes=codes, deq=deq, mag=mag)


# ----------------------------------------------------------------- layer and chain

SUB_ATTN, SUB_MLP = 0, 1
MOD_SCALE, MOD_SHIFT, MOD_GATE = 0, 1, 2
SITE_QKV, SITE_O, SITE_UP, SITE_DOWN = 0, 1, 2, 3


def _gemm_deq(a_deq, w_deq, act_scale, colscale):
    """One GEMM with scale recovery; split-K is immaterial in float64 ([notes] split-K equation)."""
    return reduce_partials((_f64(a_deq) @ _f64(w_deq))[None], act_scale, colscale)


def layer(h, x_prev, gate_prev, mod_attn, mod_mlp, w, scales, k_prefix, v_prefix,
          dims, dtype, eps, record=None, quantise_acts=True, trace=None, perturb=None):
    """One action-decoder layer.

    h: residual stream entering the layer before the previous sublayer's output is added;
    x_prev / gate_prev: the previous MLP sublayer's output and gate (None at the very
    start).  mod_attn / mod_mlp: [3][H] (scale, shift, gate).  w: dict of decoded weight
    values qkv/o/up/down ([K][N]) and colscales sqkv/so/sup/sdown (None for bf16).
    scales: the 4 static activation scales of this layer (ignored for bf16).
    Returns (h_after_attn, x_mlp, gate_mlp): the next layer adds gate_mlp * x_mlp.
    With quantise_acts=False the GEMM inputs are not rounded (calibration run) and
    record, when given, collects max|y| per site.  trace, when given, receives the
    intermediate values (residual streams, GEMM inputs as decoded codes, GEMM outputs).
    perturb, when given, is applied to every GEMM input before it is rounded; it exists
    only to measure how the chain itself amplifies tiny differences (sensitivity runs).
    """
    nh, hd = dims["n_heads"], dims["head_dim"]

    def q(v_val, site):
        if perturb is not None:
            v_val = perturb(v_val)
        if record is not None:
            record[site] = max(record.get(site, 0.0), float(np.max(np.abs(v_val))))
        if not quantise_acts:
            return _f64(v_val), 1.0
        s_a = scales[site] if dtype == "e4m3" else 1.0
        return quantise(v_val, dtype, s_a)[2], s_a

    # sublayer 1: gated residual of the previous MLP + AdaRMSNorm + quantise
    h = gated_residual(h, gate_prev, x_prev)
    y = ada_modulate(rms_normalise(h, eps), mod_attn[MOD_SCALE], mod_attn[MOD_SHIFT])
    a_qkv, s_a = q(y, SITE_QKV)
    c_qkv = _gemm_deq(a_qkv, w["qkv"], s_a, w.get("sqkv"))
    qb, kb, vb = qkv_split_bf16(c_qkv, nh, hd)
    o, _ = attention_prefix(qb, np.concatenate([_f64(k_prefix), kb]),
                            np.concatenate([_f64(v_prefix), vb]), nh, hd)
    a_o, s_a = q(o, SITE_O)
    x_attn = _gemm_deq(a_o, w["o"], s_a, w.get("so"))
    if trace is not None:
        trace.update(h_attn=h, a_qkv=a_qkv, c_qkv=c_qkv, qkv=np.concatenate([qb, kb, vb], axis=1),
                     o=o, a_o=a_o, x_attn=x_attn)
    # sublayer 2
    h = gated_residual(h, mod_attn[MOD_GATE], x_attn)
    y = ada_modulate(rms_normalise(h, eps), mod_mlp[MOD_SCALE], mod_mlp[MOD_SHIFT])
    a_up, s_a = q(y, SITE_UP)
    c_up = _gemm_deq(a_up, w["up"], s_a, w.get("sup"))
    z = silu_gate(c_up)
    a_down, s_a = q(z, SITE_DOWN)
    x_mlp = _gemm_deq(a_down, w["down"], s_a, w.get("sdown"))
    if trace is not None:
        trace.update(h_mlp=h, a_up=a_up, c_up=c_up, z=z, a_down=a_down, x_mlp=x_mlp)
    return h, x_mlp, _f64(mod_mlp[MOD_GATE])


def chain(x0, weights, scales, k_prefix, v_prefix, mod, dims, dtype, eps,
          record=None, quantise_acts=True, trace=None, perturb=None):
    """steps x layers application of ``layer`` (reading R10), then the final gated residual.

    weights: list over layers of dicts as in ``layer``; scales: [L][4]; k_prefix,
    v_prefix: [L][P][hd]; mod: [S][L][2][3][H].  Returns the residual stream after the
    last layer of the last step.  trace, when given (a dict), maps (k, l) to each
    layer's intermediates.
    """
    mod = _f64(mod)
    S, L = mod.shape[0], mod.shape[1]
    h, x_prev, gate_prev = _f64(x0), None, None
    for k in range(S):
        for l in range(L):
            h, x_prev, gate_prev = layer(h, x_prev, gate_prev, mod[k, l, SUB_ATTN],
                                         mod[k, l, SUB_MLP], weights[l], scales[l],
                                         k_prefix[l], v_prefix[l], dims, dtype, eps,
                                         record=None if record is None else record.setdefault((k, l), {}),
                                         quantise_acts=quantise_acts,
                                         trace=None if trace is None else trace.setdefault((k, l), {}),
                                         perturb=perturb)
    return gated_residual(h, gate_prev, x_prev)


def calibrate(x0_cal, weights, k_prefix, v_prefix, mod_cal, dims, eps):
    """Static activation scales from one un-quantised run on calibration inputs.

    weights: the model's master weights (decoded bf16 values; reading R13).  For every
    layer and each of its 4 GEMM-input sites, s = fp32(max |y| / 448) over every flow
    step ([notes] static-quantisation section: scales fixed ahead of the run and reused;
    weight and activation scales kept apart).  Returns [L][4].
    """
    rec = {}
    chain(x0_cal, weights, np.ones((len(weights), 4)), k_prefix, v_prefix, mod_cal, dims,
          "e4m3", eps, record=rec, quantise_acts=False)
    L = len(weights)
    amax = np.zeros((L, 4))
    for (k, l), sites in rec.items():
        for s, m in sites.items():
            amax[l, s] = max(amax[l, s], m)
    return f32(amax / codec.E4M3_MAX)


def calibrate_block(residual, x, gate, ada_scale, ada_shift, w_up, eps):
    """Static scales of a lone producer -> gate|up GEMM -> SiLU-gate block (the FP8
    single-layer and GEMM-sweep workloads) from one un-quantised run on calibration inputs.

    w_up: master weights (decoded bf16 values, [K][2F], gate | up columns; reading R13).
    Site 0 is the producer's output y = AdaRMSNorm(r + gate * x), site 1 the SiLU-gate
    output z = SiLU(y W_gate) * (y W_up) that feeds the down projection; each scale is
    fp32(max |value| / 448) ([notes] static-quantisation section).  Returns (s_y, s_z).
    """
    o = residual_norm_quant(residual, None if x is None else _f64(x)[None], None, 1.0, gate,
                            ada_scale, ada_shift, eps, "bf16", 1.0)
    z = silu_gate(o["y"] @ _f64(w_up))
    return (float(f32(np.max(np.abs(o["y"])) / codec.E4M3_MAX)),
            float(f32(np.max(np.abs(z)) / codec.E4M3_MAX)))
