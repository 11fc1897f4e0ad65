"""Seeded synthetic inputs for the action-decoder layer chain.

This module serves both the GPU library's tests/benchmark and the oracle, and holds
none of the method's arithmetic: it only draws seeded random tensors (NumPy PCG64
streams keyed by (seed, workload id, tensor id)), rounds them once to their storage
format (bfloat16 bit patterns via torch's CPU cast) and builds the conditioning
vectors.  Test inputs use seed 0, calibration inputs seed 1.

Workload recipes (shapes and distributions of the action decoder named on the pages:
action chunks of M = 10 or M = 50 rows, 18 layers x 10 flow steps):
  W1  fused residual + RMSNorm + bf16 GEMM: M=10, K=N=1024; x, r ~ N(0,1) fp32;
      gamma = 1 + 0.1 N(0,1); W ~ N(0, 1/K) bf16; eps = 1e-6.
  W2  gated MLP at M=50: W_up [1024][8192] (gate|up), W_down [4096][1024], N(0, 1/K) bf16.
  W3  FP8 path at M=10: AdaRMSNorm scale/shift/gate = c W_ada (c ~ N(0,1)^1024,
      W_ada ~ N(0, 1/1024)^(1024x3072)); W_qkv [1024][2560], W_up [1024][8192],
      W_down [4096][1024].
  W4  full chain: L layers x S steps, M=50, hidden 1024, 8 query heads, 1 KV head,
      head dim 128, 800-token bf16 prefix K/V per layer, MLP 4096.
  W5  backbone-sized sweep: K=2048, N=16384 gate|up, M in {1,10,16,32,50,64}.
"""
import numpy as np

TEST_SEED = 0
CAL_SEED = 1


def rng(seed, workload, tensor):
    return np.random.default_rng([int(seed), int(workload), int(tensor)])


def normal(seed, workload, tensor, shape, std=1.0, mean=0.0):
    """float32 N(mean, std^2) array from its own PCG64 stream."""
    g = rng(seed, workload, tensor)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return x


def to_bf16_bits(x_f32):
    """float32 array -> bfloat16 bit patterns (uint16), using torch's CPU cast (RNE)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits):
    """bfloat16 bit patterns -> float32 values (exact widening)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def weight_bf16(seed, workload, tensor, K, N):
    """W [K][N] ~ N(0, 1/K), stored as bf16 bits."""
    return to_bf16_bits(normal(seed, workload, tensor, (K, N), std=1.0 / np.sqrt(K)))


def weight_bf16_block_spread(seed, workload, tensor, K, N, spread=6, block=32):
    """W [K][N] ~ N(0, 1/K) times 2**e, one e uniform in [-spread, spread] per `block`
    consecutive k of a column (bf16 bits).  Per-block magnitudes that differ by up to
    2**(2*spread) make any mix-up between blocks and their scales visible."""
    w = normal(seed, workload, tensor, (K, N), std=1.0 / np.sqrt(K))
    e = rng(seed, workload, tensor + 1).integers(-spread, spread + 1, size=(K // block, N))
    return to_bf16_bits(w * np.repeat(np.exp2(e), block, axis=0).astype(np.float32))


def modulation(seed, workload, tensor, H, n=3):
    """[n][H] float32 conditioning outputs = c W_ada with c ~ N(0,1)^H, W_ada ~ N(0,1/H).

    Rows are (scale, shift, gate) of an AdaRMSNorm-modulated sublayer.
    """
    c = normal(seed, workload, tensor * 2, (H,)).astype(np.float64)
    w = normal(seed, workload, tensor * 2 + 1, (H, n * H), std=1.0 / np.sqrt(H)).astype(np.float64)
    return (c @ w).astype(np.float32).reshape(n, H)


# ----------------------------------------------------------------- workloads

def workload1(seed=TEST_SEED, M=10, K=1024, N=1024):
    return dict(
        x=normal(seed, 1, 0, (M, K)),
        r=normal(seed, 1, 1, (M, K)),
        gamma=normal(seed, 1, 2, (K,), std=0.1, mean=1.0),
        w=weight_bf16(seed, 1, 3, K, N),
        eps=1e-6, M=M, K=K, N=N)


def workload2(seed=TEST_SEED, M=50, K=1024, mlp=4096):
    return dict(
        x=normal(seed, 2, 0, (M, K)),
        r=normal(seed, 2, 1, (M, K)),
        w_up=weight_bf16(seed, 2, 2, K, 2 * mlp),
        w_down=weight_bf16(seed, 2, 3, mlp, K),
        eps=1e-6, M=M, K=K, mlp=mlp)


def workload3(seed=TEST_SEED, M=10, K=1024, n_qkv=2560, mlp=4096):
    return dict(
        x=normal(seed, 3, 0, (M, K)),
        r=normal(seed, 3, 1, (M, K)),
        mod=modulation(seed, 3, 2, K),
        w_qkv=weight_bf16(seed, 3, 3, K, n_qkv),
        w_up=weight_bf16(seed, 3, 4, K, 2 * mlp),
        w_down=weight_bf16(seed, 3, 5, mlp, K),
        eps=1e-6, M=M, K=K, n_qkv=n_qkv, mlp=mlp)


def chain_dims(layers=18, steps=10, M=50, hidden=1024, n_heads=8, head_dim=128,
               prefix=800, mlp=4096):
    return dict(layers=layers, steps=steps, M=M, hidden=hidden, n_heads=n_heads,
                head_dim=head_dim, prefix=prefix, mlp=mlp)


def chain_weights(dims, seed=TEST_SEED):
    """Per-layer bf16 weights and bf16 prefix K/V of the chain workload."""
    L, H = dims["layers"], dims["hidden"]
    nh, hd, P, F = dims["n_heads"], dims["head_dim"], dims["prefix"], dims["mlp"]
    nqkv = (nh + 2) * hd
    layers = []
    for l in range(L):
        t = 100 + 10 * l
        layers.append(dict(
            qkv=weight_bf16(seed, 4, t + 0, H, nqkv),
            o=weight_bf16(seed, 4, t + 1, nh * hd, H),
            up=weight_bf16(seed, 4, t + 2, H, 2 * F),
            down=weight_bf16(seed, 4, t + 3, F, H),
            k_prefix=to_bf16_bits(normal(seed, 4, t + 4, (P, hd))),
            v_prefix=to_bf16_bits(normal(seed, 4, t + 5, (P, hd)))))
    return layers


def chain_inputs(dims, seed=TEST_SEED):
    """Residual stream X0 [M][H] and the modulation table [S][L][2][3][H] of one decision.

    Flow step k has its conditioning vector c_k ~ N(0,1)^H; each (layer, sublayer) has
    its own W_ada ~ N(0, 1/H)^(H x 3H); the (scale, shift, gate) rows are c_k W_ada.
    """
    L, S, M, H = dims["layers"], dims["steps"], dims["M"], dims["hidden"]
    c = [normal(seed, 4, 20000 + k, (H,)).astype(np.float64) for k in range(S)]
    mod = np.zeros((S, L, 2, 3, H), np.float32)
    for l in range(L):
        for sub in range(2):
            w = normal(seed, 4, 30000 + 2 * l + sub, (H, 3 * H), std=1.0 / np.sqrt(H)).astype(np.float64)
            for k in range(S):
                mod[k, l, sub] = (c[k] @ w).astype(np.float32).reshape(3, H)
    return normal(seed, 4, 0, (M, H)), mod


def workload4(dims, seed=TEST_SEED, input_seed=None):
    """Full chain: X0, per-layer bf16 weights, prefix K/V (bf16), modulation table."""
    x0, mod = chain_inputs(dims, seed if input_seed is None else input_seed)
    return dict(x0=x0, layers=chain_weights(dims, seed), mod=mod, dims=dims)


def workload5(M, seed=TEST_SEED, K=2048, N=16384):
    return dict(
        x=normal(seed, 5, 0, (M, K)),
        r=normal(seed, 5, 1, (M, K)),
        w=weight_bf16(seed, 5, 2, K, N),
        eps=1e-6, M=M, K=K, N=N)
