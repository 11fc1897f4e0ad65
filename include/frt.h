/*
 * frt.h -- C ABI of the MI355X (gfx950) action-decoder layer-chain library.
 *
 * The library computes, on one GPU, the hot path the FlashRT-PAI pages describe for
 * the single-batch action decoder of a flow-matching VLA policy:
 *
 *   producer   gated residual add + (Ada)RMSNorm + static-scale quantisation, writing
 *              the next GEMM's input directly in the tile layout that GEMM reads
 *              (pages: "思考探索：具身推理加速，先看动作执行时观测有多旧", sections
 *              "CUDA Graph 与图化简分别省掉什么" -- RMSNorm and W' = diag(gamma) W
 *              equations -- and "静态量化改变了两次矩阵乘之间的工作"; rebasdaily
 *              FlashRT-PAI news summary, section "它优化的是“接力方式”": the producer's
 *              output layout is chosen so the next GEMM reads no extra data);
 *   GEMM       skinny C = A W with M <= 64 rows, split along K into FP32 partial sums
 *              (same notes, section "小 M GEMM 要看并行度，也要看归约代价", split-K
 *              equation);
 *   consumer   the next kernel reduces the FP32 partials in a fixed order, recovers the
 *              scales and carries on (norm + quantise, or SiLU gate + quantise);
 *   chain      layers x flow steps of the above, captured once into a hipGraph over
 *              persistent named buffers and replayed (same notes, section
 *              "CUDA Graph 与图化简分别省掉什么": replay reuses arguments and addresses,
 *              new inputs go into agreed buffers).
 *
 * Conventions for every entry point:
 *   - Pointers named *_dev are device pointers (hipMalloc'd or torch CUDA tensors);
 *     pointers named *_host are host pointers.  All device pointers must be 16-byte
 *     aligned.  The library never allocates device memory except the hipGraph objects
 *     owned by a chain handle; every buffer is owned by the caller.
 *   - `stream` is a hipStream_t passed as void* (NULL = the legacy default stream).
 *     Calls are asynchronous on that stream unless stated otherwise.
 *   - Every argument is validated before any HIP call: an invalid call returns an
 *     FRT_E_* code and enqueues nothing.  A failing HIP call returns FRT_E_HIP and its
 *     hipError_t is kept per thread (frt_last_hip_error).  Nothing aborts and no C++
 *     exception crosses the ABI.
 *   - Shapes: 1 <= M <= 64 action rows.  bf16 operands need K % 32 == 0, e4m3 operands
 *     K % 128 == 0; N % 16 == 0.  M is padded to Mp = 16 * ceil(M / 16) in packed
 *     operands; padding rows are written as zero codes by every producer, and no GEMM
 *     result depends on them.
 *   - Numbers: bf16 = bfloat16, round to nearest even.  e4m3 = OCP E4M3FN, round to
 *     nearest even, saturating to +-448, NaN -> 0x7F.
 */
#ifndef FRT_H
#define FRT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FRT_OK = 0,
  FRT_E_NULL = 1,       /* a required pointer is NULL                                  */
  FRT_E_SHAPE = 2,      /* M, N, K or another size out of range / not a multiple        */
  FRT_E_ALIGN = 3,      /* a device pointer is not 16-byte aligned                      */
  FRT_E_DTYPE = 4,      /* unsupported dtype / dtype combination                        */
  FRT_E_SPLITK = 5,     /* split count not in {1,2,4,8,16} or K not divisible           */
  FRT_E_WORKSPACE = 6,  /* a workspace / arena is smaller than required                 */
  FRT_E_ALIAS = 7,      /* an output overlaps an input it may not overlap               */
  FRT_E_STATE = 8,      /* handle misuse (NULL handle, unknown buffer name, ...)        */
  FRT_E_HIP = 9,        /* a HIP runtime call failed; see frt_last_hip_error()          */
  FRT_E_ARG = 10        /* another invalid argument (epilogue, layout, eps, scale)      */
} frt_status;

/* FRT_MXFP4 is a weight format only (OCP MX, FP4 E2M1 elements with one E8M0 scale per
 * 32 consecutive k of a column: 4-bit weights, the notes' "next" precision step); a GEMM
 * with MXFP4 weights takes an FRT_E4M3 operand.                                        */
typedef enum { FRT_BF16 = 1, FRT_E4M3 = 2, FRT_F32 = 3, FRT_MXFP4 = 4 } frt_dtype;

/* Logical column order of a packed weight.  FRT_W_GATE_UP pairs column tile i of the
 * gate half [0, N/2) with tile i of the up half [N/2, N) so that one workgroup holds
 * both and can apply SiLU(gate) * up in registers. */
typedef enum { FRT_W_PLAIN = 0, FRT_W_GATE_UP = 1 } frt_wlayout;

typedef enum {
  FRT_EPI_NONE = 0,            /* leave [splits][M][N] fp32 partial sums             */
  FRT_EPI_STORE_F32 = 1,       /* reduce + scale recovery, store [M][N] fp32         */
  FRT_EPI_STORE_BF16 = 2,      /* reduce + scale recovery, store [M][N] bf16 bits    */
  FRT_EPI_SILU_GATE_QUANT = 3  /* reduce + scale recovery + SiLU(gate)*up + quantise
                                  into the packed operand [Mp][N/2] of the next GEMM */
} frt_epilogue;

/* ------------------------------------------------------------------ diagnostics */
const char* frt_status_string(int status);
int frt_last_hip_error(void);      /* hipError_t of this thread's last FRT_E_HIP, else 0 */
int frt_version(void);             /* 100 * major + minor                                */
/* Enqueue n empty kernels of `workgroups` x 256 threads on `stream` (nothing is read or
 * written): the cost of a dependent launch before any work, for the launch-overlap
 * measurements (pages: rebasdaily FlashRT-PAI news summary, section "快内核为什么拼不出快
 * 管线？": the gaps between kernels are part of the pipeline's time).  Capturable into a
 * graph.  0 <= n <= 100000, 1 <= workgroups <= 65536, else FRT_E_ARG.                  */
int frt_diag_empty_kernels(void* stream, int n, int workgroups);

/* ------------------------------------------------------------------ layouts */
/* Bytes of a packed GEMM operand (A) holding M x K values: Mp * K * (2 | 1). */
size_t frt_operand_bytes(int dtype, int M, int K);
/* Bytes of a packed weight holding K x N values: K * N * (2 | 1), or for FRT_MXFP4
 * K * N / 2 code bytes + K * N / 32 scale bytes (0 unless K % 128 == 0).             */
size_t frt_weight_bytes(int dtype, int K, int N);

/* Host-only layout helpers (no HIP call; used to inspect and build test data).
 * Codes are bf16 bit patterns (uint16) or e4m3 codes (uint8), row-major logical order.
 * pack writes every byte of `packed_host` (padding rows as zero codes).              */
int frt_operand_pack_host(const void* codes_host, int dtype, int M, int K, void* packed_host);
int frt_operand_unpack_host(const void* packed_host, int dtype, int M, int K, void* codes_host);
int frt_weight_pack_host(const void* codes_host, int dtype, int K, int N, int layout,
                         void* packed_host);
int frt_weight_unpack_host(const void* packed_host, int dtype, int K, int N, int layout,
                           void* codes_host);
/* FRT_MXFP4 weights: codes [K][N] one FP4 E2M1 code per byte (low 4 bits), scale bytes
 * [K/32][N] E8M0 (block b covers k in [32b, 32b+32)).  K % 128 == 0.                  */
int frt_weight_pack_mxfp4_host(const uint8_t* codes_host, const uint8_t* scales_host, int K, int N,
                               int layout, void* packed_host);
int frt_weight_unpack_mxfp4_host(const void* packed_host, int K, int N, int layout,
                                 uint8_t* codes_host, uint8_t* scales_host);

/* ------------------------------------------------------------------ offline weight prep */
/* Pack a bf16 weight W [K][N] (row-major bits, device) for the skinny GEMM.
 * gamma_dev [K] fp32 or NULL: fold a fixed RMSNorm gain into the weight,
 *   W' = diag(gamma) W (notes, section "CUDA Graph 与图化简分别省掉什么", W' equation),
 *   computed in fp32 and rounded once to the target format.
 * dtype FRT_BF16: packed bf16 of W'.  colscale_dev ignored (may be NULL).
 * dtype FRT_E4M3: per-output-channel scale s_w[n] = max_k |W'[k][n]| / 448 written to
 *   colscale_dev [N] (fp32); codes e4m3(W'[k][n] / s_w[n]); a zero column gets s_w = 0
 *   and zero codes (the notes' static-quantisation section keeps weight scales apart
 *   from activation scales).
 * dtype FRT_MXFP4: each block of 32 consecutive k of a column (k in [32b, 32b+32)) gets
 *   the E8M0 scale X = 2^e, e = floor(log2 max|W'|) - 2 (the largest FP4 E2M1 magnitude
 *   is 6 = 1.5 * 2^2), clamped to [-127, 127]; elements are FP4 E2M1 codes of W' / X,
 *   rounded to nearest even and saturated at +-6; an all-zero block gets scale byte 0
 *   and zero codes (OCP Microscaling Formats v1.0: MXFP4).  No column scale (colscale_dev
 *   ignored); K % 128 == 0.
 * layout: FRT_W_PLAIN or FRT_W_GATE_UP (N % 32 == 0).  w_packed_dev must hold
 * frt_weight_bytes(dtype, K, N) bytes and must not overlap w_bf16_dev.              */
int frt_pack_weight(void* stream, int K, int N, const uint16_t* w_bf16_dev,
                    const float* gamma_dev, int dtype, int layout, void* w_packed_dev,
                    float* colscale_dev);

/* ------------------------------------------------------------------ producer */
/* Gated residual + (Ada)RMSNorm + static-scale quantisation, one fused kernel.
 *
 *   x[m][k]  = (sum_{j=0..x_splits-1} x_dev[j][m][k]) * x_scale * x_colscale[k]
 *              (partials summed in ascending j; x_colscale NULL = 1; x_dev NULL = no x)
 *   h        = residual + gate[k] * x          (gate NULL = 1)
 *   xhat     = h / sqrt(mean_k(h^2) + eps)     (notes, RMSNorm equation)
 *   y        = xhat * (1 + ada_scale[k]) + ada_shift[k]   (NULL = 0; AdaRMSNorm)
 *   operand  = bf16(y)  or  e4m3(y / act_scale)           (packed, Mp x K)
 *
 * x_dev [x_splits][M][K] fp32, residual_dev [M][K] fp32, residual_out_dev [M][K] fp32
 * (NULL = h not stored; may equal residual_dev for an in-place update); vectors [K]
 * fp32.  operand_out_dev: frt_operand_bytes(out_dtype, M, K) bytes, or NULL to only
 * update the residual stream.  act_scale > 0 (used for FRT_E4M3 only).
 * 1 <= x_splits <= 16; K % 32 (bf16) or % 128 (e4m3); K <= 4096; eps >= 0.           */
int frt_residual_norm_quant(void* stream, int M, int K,
                            const float* x_dev, int x_splits, float x_scale,
                            const float* x_colscale_dev,
                            const float* residual_dev, float* residual_out_dev,
                            const float* gate_dev, const float* ada_scale_dev,
                            const float* ada_shift_dev, float eps,
                            int out_dtype, float act_scale, void* operand_out_dev);

/* ------------------------------------------------------------------ skinny GEMM */
/* C = A W with A the packed operand [Mp][K] and W the packed weight [K][N], both
 * FRT_BF16 or both FRT_E4M3, or (ab_dtype FRT_MXFP4) MXFP4 weights with an FRT_E4M3
 * operand (block-scaled FP4 x FP8 MFMA), all with fp32 accumulation.  bf16 products are
 * exact; e4m3 x e4m3 products are exact for M <= 16 (codes widened to bf16) and go through
 * the fp8 MFMA above that, whose internal sums keep about 13 bits (partials within about
 * 1.5e-5 relative of the exact products).  K is cut into `splits` contiguous equal chunks;
 * chunk j's product is partial P_j (notes, split-K equation).
 *
 * splits: 1, 2, 4, 8 or 16, or 0 to let the library choose for (M, N, K, dtype).
 * partials_dev [splits][M][N] fp32 workspace, partials_bytes >= splits*M*N*4; it may be
 *   NULL (bytes 0) only when splits resolves to 1 and epi != FRT_EPI_NONE.
 * Scale recovery: C = (sum_j P_j) * act_scale * w_colscale[n] (w_colscale NULL = 1).
 * epi FRT_EPI_NONE: the partials are the result (a consumer reduces them later).
 * epi STORE_F32 / STORE_BF16: out_dev [M][N].
 * epi SILU_GATE_QUANT: needs layout FRT_W_GATE_UP; z = SiLU(C[:, :N/2]) * C[:, N/2:],
 *   out_dev = packed operand of z (out_dtype FRT_BF16 or FRT_E4M3 with out_act_scale),
 *   frt_operand_bytes(out_dtype, M, N/2) bytes.
 * With splits == 1 the epilogue runs inside the GEMM kernel; otherwise a second
 * (consumer) kernel reduces the partials in ascending j.                             */
int frt_skinny_gemm_splitk(void* stream, int M, int N, int K, int splits,
                           int ab_dtype, int layout, const void* a_packed_dev,
                           const void* w_packed_dev, const float* w_colscale_dev,
                           float act_scale, float* partials_dev, size_t partials_bytes,
                           int epi, void* out_dev, int out_dtype, float out_act_scale);

/* Allocation-free variant of frt_skinny_gemm_splitk, for callers that cannot allocate
 * device memory (code under hipGraph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments and results as frt_skinny_gemm_splitk with an epilogue
 * (epi STORE_F32, STORE_BF16 or SILU_GATE_QUANT; FRT_E_ARG for FRT_EPI_NONE, whose
 * partials are the caller's output), minus the partials workspace: when splits resolves
 * to more than 1, the [splits][M][N] fp32 partials go to a scratch array inside the
 * library, one per GPU, of frt_noalloc_scratch_bytes() bytes (16 MiB), held from the first
 * call on that GPU until the process ends.  splits * M * N * 4 above that size returns
 * FRT_E_WORKSPACE before anything is enqueued.  The call allocates nothing.  Every call on
 * one GPU shares that GPU's array, so calls that overlap in time on one GPU (different
 * streams, different threads) race and must be ordered by the caller; each call fully
 * rewrites the partials it reads.                                                       */
int frt_skinny_gemm_splitk_noalloc(void* stream, int M, int N, int K, int splits,
                                   int ab_dtype, int layout, const void* a_packed_dev,
                                   const void* w_packed_dev, const float* w_colscale_dev,
                                   float act_scale, int epi, void* out_dev, int out_dtype,
                                   float out_act_scale);
size_t frt_noalloc_scratch_bytes(void);

/* Split-K consumer on its own: reduce [splits][M][N] partials (ascending j), recover
 * scales, then apply `epi` (STORE_F32, STORE_BF16 or SILU_GATE_QUANT; for the latter
 * the columns are in logical order, gate = [0, N/2)).                                */
int frt_splitk_reduce(void* stream, int M, int N, int splits, const float* partials_dev,
                      float act_scale, const float* w_colscale_dev, int epi, void* out_dev,
                      int out_dtype, float out_act_scale);

/* Library's split-K choice for a GEMM whose fp32 partials are its output (FRT_EPI_NONE;
 * what splits = 0 resolves to there).  With an epilogue, splits = 0 resolves to 1: a
 * split would cost a separate consumer kernel.  0 for an unsupported shape.            */
int frt_splitk_choose(int M, int N, int K, int ab_dtype);

/* Fused QKV projection: the skinny GEMM of a [Mp][K] operand with a packed weight of
 * N = (n_heads + 2) * head_dim columns [Q | K | V] (three projections of one input merged
 * into one wider GEMM: notes, section "CUDA Graph 与图化简分别省掉什么"), reduced (ascending
 * split), scale-recovered (act_scale * w_colscale[n]) and rounded to bf16, then written
 * straight where attention reads it: q_out_dev [M][n_heads*head_dim] and k_out_dev
 * [M][head_dim] row-major; V transposed, v_t_out_dev[d * v_ld + m] (typically k_out_dev =
 * row prefix_len of a key cache and v_t_out_dev = column prefix_len of a transposed value
 * cache).  splits as for frt_skinny_gemm_splitk; partials_dev [splits][M][N] fp32 is
 * needed only when splits resolves to more than 1.  head_dim % 16 == 0, v_ld >= M;
 * v_t_out_dev needs only 2-byte alignment (it is written element by element).           */
int frt_skinny_gemm_qkv(void* stream, int M, int K, int n_heads, int head_dim, int splits,
                        int ab_dtype, const void* a_packed_dev, const void* w_packed_dev,
                        const float* w_colscale_dev, float act_scale, float* partials_dev,
                        size_t partials_bytes, uint16_t* q_out_dev, uint16_t* k_out_dev,
                        uint16_t* v_t_out_dev, int v_ld);

/* ------------------------------------------------------------------ attention */
/* Attention of the M action rows over a cached key/value sequence: one KV head shared by
 * n_heads query heads, no mask, scale 1/sqrt(head_dim).  Not on the pages; it is the
 * step between the QKV and O GEMMs of the action-decoder layer.
 *   q_dev [M][n_heads*head_dim] bf16; k_dev [kv_len][head_dim] bf16 (the cached prefix
 *   followed by the M own rows, kv_len = prefix_len + M); v_t_dev [head_dim][ldv] bf16,
 *   the values transposed (key index contiguous), ldv a multiple of 32 >= kv_len
 *   (elements past kv_len are read but never used);
 *   O[m][h*d + e] = softmax_t(q_h . k_t / sqrt(d)) v_t[e], fp32-accurate;
 *   operand_out = packed bf16(O) or e4m3(O / out_act_scale), Mp x n_heads*head_dim.
 * Short sequences run as one workgroup per (head, 16-row block); long ones are cut into
 * 128-key chunks (64-key chunks when that would leave fewer than 128 workgroups) whose
 * FP32 partials (max, sum, unnormalised output) a second kernel
 * merges in chunk order (deterministic).
 * workspace_dev: frt_attention_workspace_bytes(...) bytes, no initial contents needed;
 * calls that share a workspace must not overlap in time.
 * head_dim == 128, 1 <= n_heads <= 16, M <= kv_len <= 8192 + 64.                        */
size_t frt_attention_workspace_bytes(int M, int n_heads, int head_dim, int kv_len);
int frt_attention_prefix(void* stream, int M, int n_heads, int head_dim, int kv_len,
                         const uint16_t* q_dev, const uint16_t* k_dev, const uint16_t* v_t_dev,
                         int ldv, int out_dtype, float out_act_scale, void* operand_out_dev,
                         void* workspace_dev, size_t workspace_bytes);

/* ------------------------------------------------------------------ layer chain */
/* One action-decoder layer (per layer l, per flow step k):
 *   h   = h + gate_mlp(prev) * x_mlp(prev)             (previous layer's MLP output)
 *   a   = quant(AdaRMSNorm(h; mod[k][l][0]))           producer
 *   q, k_cache[l][P..], v_cache[l][..][P..] = bf16(a W_qkv[l])   GEMM (split-K), own rows
 *   o   = quant(attention(q, k_cache[l], v_cache[l]))  over prefix + own rows
 *   x   = o W_o[l];  h = h + mod[k][l][0].gate * x     GEMM, then producer
 *   b   = quant(AdaRMSNorm(h; mod[k][l][1]))
 *   z   = quant(SiLU(b W_gate) * (b W_up))             GEMM + fused consumer
 *   x_mlp = z W_down[l]                                GEMM; reduced by the next producer
 * Flow steps compose: the residual stream leaving step k enters step k+1; after the
 * last layer of the last step a final producer adds the last MLP output into "x".
 * mod rows are (scale, shift, gate); the producer that starts layer l uses layer l's
 * modulation while reducing layer l-1's output (next-layer conditioning prepares the
 * next input: notes, static-quantisation section).
 * When the key axis is cut into chunks (prefix_len + M > 128 keys at most 16 chunks) and
 * hidden % 256 == 0, the attention merge runs inside the O projection: one kernel
 * merges a head's chunk partials and multiplies the head output by that head's rows of
 * W_o, so the O projection is split by head (splits_o resolves to n_heads; an explicit
 * other value keeps the two apart).  Without debug buffers this saves one kernel per
 * layer; with them the two run apart with the same split, and the results are bitwise
 * the same.                                                                           */
typedef struct frt_chain_desc {
  int layers, steps, M, hidden, n_heads, head_dim, prefix_len, mlp;
  int dtype;                 /* FRT_BF16 or FRT_E4M3 (weights and GEMM inputs), or
                                FRT_MXFP4 (MXFP4 weights, FRT_E4M3 GEMM inputs)         */
  float eps;
  int splits_qkv, splits_o, splits_up, splits_down;   /* 0 = library choice            */
  int use_graph;             /* 1: capture once, replay with one hipGraphLaunch          */
  int keep_intermediates;    /* 1: every (step, layer) writes its own debug buffers      */
  int prefetch_next;         /* 1: each producer also reads the weights of a GEMM that
                                follows it ahead (the first the QKV weights, the second
                                the down projection's), from extra workgroups on the XCDs
                                that will stream them, so the GEMM finds them in L2 (the
                                launch-overlap analogue).  Results are bitwise unchanged. */
  /* host arrays of `layers` device pointers to packed weights (frt_pack_weight):
   * qkv [hidden][(n_heads+2)*head_dim] plain, o [n_heads*head_dim][hidden] plain,
   * up [hidden][2*mlp] FRT_W_GATE_UP, down [mlp][hidden] plain.                        */
  const void* const* w_qkv;
  const void* const* w_o;
  const void* const* w_up;
  const void* const* w_down;
  /* e4m3 only: host arrays of `layers` device pointers to fp32 column scales. */
  const float* const* s_qkv;
  const float* const* s_o;
  const float* const* s_up;
  const float* const* s_down;
} frt_chain_desc;

typedef struct frt_chain frt_chain;

/* Bytes of device memory the chain needs in the caller's arena (named buffers,
 * operands, partials; plus debug buffers when keep_intermediates).  0 on bad desc.   */
size_t frt_layer_chain_arena_bytes(const frt_chain_desc* desc);
/* Bind the named buffers inside `arena_dev` (16-byte aligned, >= arena_bytes) and,
 * with use_graph, capture the whole chain on `capture_stream` (synchronous). */
int frt_layer_chain_create(const frt_chain_desc* desc, void* arena_dev, size_t arena_bytes,
                           void* capture_stream, frt_chain** out);
/* Device address and size of a named buffer:
 *   "x_in"      [M][hidden] fp32   residual stream entering the first layer of the first step
 *   "x_out"     [M][hidden] fp32   residual stream after the last layer of the last step
 *   "mod"       [steps][layers][2][3][hidden] fp32   (scale, shift, gate) per sublayer
 *   "act_scale" [layers][4] fp32   static activation scales (e4m3): qkv, o, up, down inputs
 *   "k_cache"   [layers][prefix_len + M][head_dim] bf16 and
 *   "v_cache"   [layers][head_dim][ldv] bf16 (values transposed, ldv = prefix_len + M
 *               rounded up to 32): the caller writes the prefix keys / values [0,
 *               prefix_len); the entries after them are each layer's own rows, rewritten
 *               by its QKV GEMM at every step
 *   "h"         [M][hidden] fp32   working residual stream (not kept per layer)
 *   debug (keep_intermediates): "dbg_h_attn", "dbg_h_mlp" [steps][layers][M][hidden] fp32,
 *   "dbg_a_qkv", "dbg_a_o", "dbg_a_up", "dbg_a_down" [steps][layers] packed operands,
 *   "dbg_p_o", "dbg_p_down" [steps][layers][splits][M][N] fp32, "dbg_q"
 *   [steps][layers][M][n_heads*head_dim] bf16, and "dbg_k_own", "dbg_v_own"
 *   [steps][layers][M][head_dim] bf16 (each layer-step's own key and value rows, copied
 *   out of the caches by one extra kernel per layer before the next step rewrites them);
 *   each (step, layer) slice starts on a 256-byte boundary.  A name whose buffer is
 *   empty returns FRT_E_STATE.                                                         */
int frt_layer_chain_buffer(frt_chain* chain, const char* name, void** dev, size_t* bytes);
/* Static activation scales for an e4m3 chain built from the same bf16 master weights:
 * runs this bf16 chain once, eagerly, on the current "x_in" / "mod" / caches (the
 * calibration inputs), records max |value| at every GEMM-input site (qkv, o, up, down of
 * each layer, over every flow step) before its bf16 rounding, and writes
 * scales_dev[l*4 + site] = max / 448 (fp32, device, [layers][4]).  The scales are then
 * fixed for every later run (notes, section "静态量化改变了两次矩阵乘之间的工作": scales
 * fixed ahead of the run, weight and activation scales kept apart).  Also writes
 * "x_out" like a run.  FRT_E_DTYPE unless the chain is bf16.                          */
int frt_layer_chain_calibrate(frt_chain* chain, void* stream, float* scales_dev);

/* Execution-state capsule (abstract page, "execution-state capsule": the state a
 * decision runs on is captured as a unit that can be restored or forked).  The chain's
 * persistent state -- "x_in", "x_out", "mod", "act_scale", "k_cache", "v_cache" -- is the
 * leading region of the arena.  A capsule is that region followed by a 256-byte trailer
 * (a magic word and a token of the chain's shape fields and state layout); state_bytes
 * counts both.
 *   snapshot: chain state -> capsule_dev, then the trailer (queued on `stream`,
 *             asynchronous);
 *   restore:  reads the capsule's trailer back after the work already queued on
 *             `stream`, waits for it (synchronous with the host, so not capturable), and
 *             returns FRT_E_STATE unless the capsule was written by a chain with the same
 *             shape fields (layers, steps, M, hidden, n_heads, head_dim, prefix_len, mlp,
 *             activation format: bf16, or e4m3 for e4m3 and MXFP4 weights); then queues
 *             the copy capsule_dev -> chain state on `stream`.
 * Restoring a capsule into a second chain of the same shape forks the state (that chain
 * may hold other weights).  capsule_dev is caller-owned device memory, 16-byte aligned,
 * exactly state_bytes long (FRT_E_WORKSPACE otherwise), and must not overlap the arena
 * (FRT_E_ALIAS).  The rest of the arena (working buffers) is rewritten by every run and
 * is not part of the state.                                                           */
size_t frt_layer_chain_state_bytes(const frt_chain* chain);
int frt_layer_chain_snapshot(frt_chain* chain, void* stream, void* capsule_dev, size_t capsule_bytes);
int frt_layer_chain_restore(frt_chain* chain, void* stream, const void* capsule_dev, size_t capsule_bytes);

/* Run every step and layer once on `stream` (one hipGraphLaunch, or eager launches). */
int frt_layer_chain_run(frt_chain* chain, void* stream);
/* Kernels one run launches (graph nodes when captured). */
int frt_layer_chain_kernel_count(const frt_chain* chain);
int frt_layer_chain_destroy(frt_chain* chain);

#ifdef __cplusplus
}
#endif
#endif /* FRT_H */
