// Attention of the M action rows over a cached bf16 key/value sequence (the prefix
// followed by the M own rows), writing the packed operand of the O projection.
//
// This step is not on the pages; it links the QKV-merged GEMM (observation-age notes
// "思考探索：具身推理加速，先看动作执行时观测有多旧", section "CUDA Graph 与图化简分别省掉什么":
// three projections of one input become one wider GEMM) to the O projection.  Its
// structure follows the notes' split-K section ("小 M GEMM 要看并行度，也要看归约代价"):
// the key axis is cut into chunks that run as separate workgroups, each leaves an FP32
// partial (max, sum and unnormalised output), and a consumer kernel merges the partials
// in chunk order and carries on into quantisation.  (Merging inside the same kernel by
// the last workgroup to arrive needs a device-scope release/acquire per workgroup, which
// writes back and invalidates L2 and cost far more than a second kernel.)
//
// Keys and values live in a per-layer cache: K row-major [kv_len][128], V transposed
// [128][ldv] (key index contiguous) so that every MFMA operand is one contiguous load.  Scores are bf16 x bf16
// MFMAs (exact products, fp32 sums); probabilities multiply V as three bf16 pieces
// (hi + mid + lo carry all 24 bits of the fp32 value), so the output is fp32-accurate.
#include "gemm_kernel.hpp"

#include <stdlib.h>

namespace frt {

constexpr int HD = 128;

__device__ __forceinline__ bf16x8 bf16x8_from(const uint32_t* w4) {
  u32x4 v = {w4[0], w4[1], w4[2], w4[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Workspace layout (only when the key axis is cut into more than one chunk):
// [chunks][heads][MB] partial records of (16 (m, l) pairs | 16*128 O) fp32, each row's
// running maximum m and sum l side by side so a reader takes both with one 8-byte load.
__host__ __device__ inline size_t attn_record_floats() { return 32 + 16 * HD; }

// Keys per workgroup.  Measured on MI355X (850 keys): one 32-key block per wave, merged
// by a second kernel, beats whole-sequence workgroups whose waves walk several blocks in
// turn (each block then pays its own load latency, and one CU fetches every key and value
// line of the sequence).  128-key chunks of 4 waves are fastest while they give at least
// 128 workgroups (M = 50: 34.5 us/layer against 36.1 with 64-key chunks); below that,
// 64-key chunks of 2 waves spread the work wider (M = 10: 29.6 against 30.2).  A
// sequence that fits one chunk needs no merge.  FRT_ATTN_CHUNK_KEYS (64, 128, 256, 512 or
// 1024) overrides the choice for tuning; chunks of 256 and more use 8 waves.
int attention_chunk_keys(int M, int n_heads, int kv_len) {
  static int env = -1;
  if (env < 0) {
    const char* e = getenv("FRT_ATTN_CHUNK_KEYS");
    env = e ? atoi(e) : 0;
    if (env != 64 && env != 128 && env != 256 && env != 512 && env != 1024) env = 0;
  }
  if (env > 0) return env;
  const int wgs128 = n_heads * ((M + 15) / 16) * ((kv_len + 127) / 128);
  return wgs128 < 128 && kv_len > 64 ? 64 : 128;
}
size_t attention_workspace_bytes(int M, int n_heads, int kv_len) {
  const int MB = (M + 15) / 16, ck = attention_chunk_keys(M, n_heads, kv_len), nch = (kv_len + ck - 1) / ck;
  return nch > 1 ? (size_t)nch * n_heads * MB * attn_record_floats() * 4 : 16;
}

// One 32-key block's operands for one wave: K rows (MFMA A operand of S^T = K Q^T) and
// V^T columns (MFMA A operand of O^T = V^T P^T).  Accumulator row r (r = 4g + i, i < 4)
// of score tile hf holds key t0 + 8g + 4hf + i: the K operand's row r is loaded from that
// key, so the 8 probabilities that lane group g = L/16 holds after the scores (rows 4g..4g+3
// of both tiles) are the contiguous keys t0 + 8g + [0, 8), exactly the k slots of the P^T
// operand of that lane group.  Each lane's V^T operand is then one contiguous 16-byte load
// (keys t0 + 8g + [0, 8) of column d = 16*dt + L%16) and P^T needs no shuffle.  Measured on
// MI355X (M=50 bf16 chain, paired): 29.90 -> 29.57 us/layer against two 8-byte V loads.
struct KVBlock {
  u32x4 k[2][4];
  u32x4 v[8];
};

__device__ __forceinline__ void load_block(KVBlock& b, const AttnParams& p, int t0, int lane) {
  const int g4 = lane >> 4, q = lane & 15, T = p.kv_len;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int t = t0 + 8 * (q >> 2) + 4 * hf + (q & 3);
    const uint16_t* krow = p.k + (size_t)(t < T ? t : T - 1) * HD + 8 * g4;  // clamped, masked later
#pragma unroll
    for (int dc = 0; dc < 4; ++dc) b.k[hf][dc] = *reinterpret_cast<const u32x4*>(krow + 32 * dc);
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)  // rows padded to whole 32-key blocks
    b.v[dt] = *reinterpret_cast<const u32x4*>(p.vt + (size_t)(16 * dt + q) * p.ldv + t0 + 8 * g4);
}

// Online-softmax update of one wave's state with one 32-key block.
__device__ __forceinline__ void attend_block(const KVBlock& b, const bf16x8 (&qf)[4], int t0, int lane, int T,
                                             float& m_run, float& l_run, f32x4 (&o)[8]) {
  const int g4 = lane >> 4;
  const float NEG_INF = -__builtin_huge_valf();
  // keys past the sequence were loaded from its last row (finite), and their scores are
  // replaced by -inf below, so the K operand needs no masking
  f32x4 s[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    s[hf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dc = 0; dc < 4; ++dc)
      s[hf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b.k[hf][dc]), qf[dc], s[hf], 0, 0, 0);
  }
  // s[hf][r] = score of key t0 + 8*(L/16) + 4*hf + r for query L%16, kept in base-2
  // units (scaled by log2(e) / sqrt(128)) so every exponential is one hardware exp2;
  // maxima and the merge weights below use the same units
  const float scale = 0.08838834764831845f * 1.4426950408889634f;
  float bmax = NEG_INF;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s[hf][r] = t0 + 8 * g4 + 4 * hf + r < T ? s[hf][r] * scale : NEG_INF;
      bmax = fmaxf(bmax, s[hf][r]);
    }
  bmax = xor_max<16>(bmax);
  bmax = xor_max<32>(bmax);
  const float m_new = fmaxf(m_run, bmax);  // finite: the block holds a key < T
  const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
  float pr[8];
  float psum = 0.f;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pr[4 * hf + r] = __builtin_amdgcn_exp2f(s[hf][r] - m_new);
      psum += pr[4 * hf + r];
    }
  l_run = l_run * alpha + psum;
  m_run = m_new;
  // P^T (MFMA B operand) as three bf16 pieces that carry the fp32 value exactly; pr[j] is
  // key t0 + 8*(L/16) + j, the lane's k slot j
  uint32_t hi[4], mid[4], lo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float a0 = pr[2 * j], a1 = pr[2 * j + 1];
    hi[j] = bf16_pack2(a0, a1);
    a0 -= bf16_to_f32(hi[j]);
    a1 -= bf16_to_f32(hi[j] >> 16);
    mid[j] = bf16_pack2(a0, a1);
    a0 -= bf16_to_f32(mid[j]);
    a1 -= bf16_to_f32(mid[j] >> 16);
    lo[j] = bf16_pack2(a0, a1);
  }
  const bf16x8 phi = bf16x8_from(hi), pmid = bf16x8_from(mid), plo = bf16x8_from(lo);
  // keys past the sequence: zero their V entries (the clamped or padded loads are finite
  // or not, and 0 * NaN would poison the sum)
  const bool vok = t0 + 8 * g4 + 7 < T;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    uint32_t vw[4] = {b.v[dt].x, b.v[dt].y, b.v[dt].z, b.v[dt].w};
    if (!vok) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (t0 + 8 * g4 + j >= T) vw[j >> 1] &= (j & 1) ? 0x0000ffffu : 0xffff0000u;
    }
    const bf16x8 vf = bf16x8_from(vw);
    o[dt] *= alpha;
    o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, phi, o[dt], 0, 0, 0);
    o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pmid, o[dt], 0, 0, 0);
    o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, plo, o[dt], 0, 0, 0);
  }
}

// Workgroup = (query head h, 16-row block mb, key chunk c); its NW waves take interleaved
// 32-key blocks of the chunk, each keeping an online softmax with the next block's loads
// in flight while the current one is computed; the waves merge in wave order.  With one
// chunk the workgroup writes the quantised output, otherwise an fp32 partial record.
template <int NW, bool MULTI, bool REC, int ODT>
__global__ void __launch_bounds__(64 * NW) attn_chunk_kernel(const AttnParams p) {
  const int h = blockIdx.x, mb = blockIdx.y, ch = blockIdx.z;
  // wave index made provably uniform: MFMAs ignore EXEC, so branches around them must be
  // scalar branches
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int M = p.M, T = p.kv_len, nq = p.n_heads * HD, MB = gridDim.y;
  const int g4 = lane >> 4, q = lane & 15;
  const int c0 = ch * p.chunk_keys;
  const int c1 = min(T, c0 + p.chunk_keys);
  const int nblk = (c1 - c0 + 31) / 32;

  __shared__ f32x4 comb[NW][8][64];
  __shared__ float cm[NW][16], cl[NW][16];

  const float NEG_INF = -__builtin_huge_valf();
  float m_run = NEG_INF, l_run = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (wave < nblk) {
    // padding query rows (mq >= M) attend with row 0's query: finite, and their outputs
    // are written as zero codes
    const int mq = mb * 16 + q;
    const uint16_t* qrow = p.q + (size_t)(mq < M ? mq : 0) * nq + h * HD + 8 * g4;
    bf16x8 qf[4];
#pragma unroll
    for (int dc = 0; dc < 4; ++dc) qf[dc] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + 32 * dc));
    KVBlock cur;
    load_block(cur, p, c0 + 32 * wave, lane);
    if constexpr (!MULTI) {
      // every load of the wave (Q, K and V) goes out before the first MFMA waits: left to
      // itself the compiler issued the V loads after the first Q.K^T MFMAs, a memory round
      // trip after the others (measured on MI355X, paired, bitwise equal outputs: -0.05 us
      // per layer at M=50 in bf16, e4m3 and MXFP4, -0.02 to -0.05 at M=10)
      __builtin_amdgcn_sched_barrier(0);
      attend_block(cur, qf, c0 + 32 * wave, lane, T, m_run, l_run, o);  // one block per wave
    } else {
      KVBlock nxt;
      for (int bi = wave; bi < nblk; bi += 2 * NW) {
        const bool more = bi + NW < nblk;
        if (more) load_block(nxt, p, c0 + 32 * (bi + NW), lane);
        attend_block(cur, qf, c0 + 32 * bi, lane, T, m_run, l_run, o);
        if (more) {
          if (bi + 2 * NW < nblk) load_block(cur, p, c0 + 32 * (bi + 2 * NW), lane);
          attend_block(nxt, qf, c0 + 32 * (bi + NW), lane, T, m_run, l_run, o);
        }
      }
    }
    l_run = xor_add<16>(l_run);
    l_run = xor_add<32>(l_run);
  }

  // ---- merge the waves (wave order)
  if (lane < 16) {
    cm[wave][lane] = m_run;
    cl[wave][lane] = l_run;
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) comb[wave][dt][lane] = o[dt];
  __syncthreads();
  // thread -> (query row tq, consecutive d); 64*NW threads cover 16 x 128
  constexpr int DPT = 128 * 16 / (64 * NW);   // d per thread: 8 (4 waves) or 4 (8 waves)
  const int tq = threadIdx.x / (128 / DPT);
  const int d0 = (threadIdx.x % (128 / DPT)) * DPT;
  float mx = NEG_INF;
  for (int w = 0; w < NW; ++w) mx = fmaxf(mx, cm[w][tq]);
  float wgt[NW], den = 0.f;
  for (int w = 0; w < NW; ++w) {
    wgt[w] = cm[w][tq] == NEG_INF ? 0.f : __builtin_amdgcn_exp2f(cm[w][tq] - mx);
    den += wgt[w] * cl[w][tq];
  }
  float* rec = p.workspace + (((size_t)ch * p.n_heads + h) * MB + mb) * attn_record_floats();
  const float os = load_scale(p.out_scale_ptr, p.out_scale);
  const int m = mb * 16 + tq;
#pragma unroll
  for (int e4 = 0; e4 < DPT; e4 += 4) {
    const int d = d0 + e4, dt = d >> 4, lg = (d & 15) >> 2;   // 4 d sit in one accumulator of one lane
    f32x4 acc = comb[0][dt][lg * 16 + tq] * wgt[0];
    for (int w = 1; w < NW; ++w) acc += comb[w][dt][lg * 16 + tq] * wgt[w];
    if constexpr (!REC) {
      const f32x4 ov = acc * (1.0f / den);
      store_operand4(p.operand, ODT, MB, m, h * HD + d, ov.x, ov.y, ov.z, ov.w, os, m >= M);
      if (m < M) record_amax(p.amax, ov.x, ov.y, ov.z, ov.w);
    } else if (m < M) {  // padding rows' records are never read
      *reinterpret_cast<f32x4*>(rec + 32 + tq * HD + d) = acc;
    }
  }
  if (REC && m < M && (threadIdx.x % (128 / DPT)) == 0) {
    *reinterpret_cast<u32x2*>(rec + 2 * tq) = u32x2{__float_as_uint(mx), __float_as_uint(den)};
  }
}

// Merge of the chunk records of (head h, 16-row block mb) for one thread: query row tq,
// d0 .. d0+7; chunks in order (deterministic).  A padding row (live = false) has no
// records (the chunk kernel writes none) and merges to zeros, which are written as zero
// codes.  With CH > 0 (nch <= CH) every record of
// the thread is loaded before the first is used, so the records, written by the previous
// kernel on other XCDs, cost one memory latency instead of one per chunk; slots past the
// last chunk load chunk 0 again (always valid) and weigh it 0.  Maxima are in base-2
// units (see attend_block).
template <int CH>
__device__ __forceinline__ void merge_records(const AttnParams& p, int h, int mb, int MB, int nch, int tq, int d0,
                                              bool live, float (&o)[8]) {
  if (!live) {
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
    return;
  }
  const float NEG_INF = -__builtin_huge_valf();
  const float* rec0 = p.workspace + ((size_t)h * MB + mb) * attn_record_floats();
  const size_t cstride = (size_t)p.n_heads * MB * attn_record_floats();
  float mx = NEG_INF, den = 0.f, num[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add = [&](float mc, float lc, f32x4 a, f32x4 b) {
    const float wc = mc == NEG_INF ? 0.f : __builtin_amdgcn_exp2f(mc - mx);
    den += wc * lc;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      num[e] += wc * a[e];
      num[4 + e] += wc * b[e];
    }
  };
  if constexpr (CH > 0) {
    float mc[CH], lc[CH];
    f32x4 a[CH], b[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const float* rc = rec0 + (c < nch ? c : 0) * cstride;
      const u32x2 ml = *reinterpret_cast<const u32x2*>(rc + 2 * tq);
      mc[c] = __uint_as_float(ml.x);
      lc[c] = __uint_as_float(ml.y);
      a[c] = *reinterpret_cast<const f32x4*>(rc + 32 + tq * HD + d0);
      b[c] = *reinterpret_cast<const f32x4*>(rc + 32 + tq * HD + d0 + 4);
    }
    __builtin_amdgcn_sched_barrier(0);  // every record load issued before the first wait
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (c >= nch) mc[c] = NEG_INF;
      mx = fmaxf(mx, mc[c]);
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) add(mc[c], lc[c], a[c], b[c]);
  } else {
    for (int c = 0; c < nch; ++c) mx = fmaxf(mx, rec0[c * cstride + 2 * tq]);
    for (int c = 0; c < nch; ++c) {
      const float* rc = rec0 + c * cstride;
      add(rc[2 * tq], rc[2 * tq + 1], *reinterpret_cast<const f32x4*>(rc + 32 + tq * HD + d0),
          *reinterpret_cast<const f32x4*>(rc + 32 + tq * HD + d0 + 4));
    }
  }
  const float rden = 1.0f / den;  // one division; the products are within an ulp of the quotients
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = num[e] * rden;
}

// Merge kernel: workgroup = (head h, 16-row block mb); thread -> (query row, 8 d).
template <int CH, int ODT>
__global__ void __launch_bounds__(256) attn_combine_kernel(const AttnParams p, int nch) {
  const int h = blockIdx.x, mb = blockIdx.y, MB = gridDim.y;
  const int tq = threadIdx.x >> 4;
  const int d0 = (threadIdx.x & 15) * 8;
  float o[8];
  merge_records<CH>(p, h, mb, MB, nch, tq, d0, mb * 16 + tq < p.M, o);
  const float os = load_scale(p.out_scale_ptr, p.out_scale);
  const int m = mb * 16 + tq;
  const int k = h * HD + d0;
  store_operand4(p.operand, ODT, MB, m, k, o[0], o[1], o[2], o[3], os, m >= p.M);
  store_operand4(p.operand, ODT, MB, m, k + 4, o[4], o[5], o[6], o[7], os, m >= p.M);
  if (m < p.M) {
    record_amax(p.amax, o[0], o[1], o[2], o[3]);
    record_amax(p.amax, o[4], o[5], o[6], o[7]);
  }
}

// The merge fused with the O projection (the chain, when the key axis is split):
// workgroup = (head h, 16-row block mb, column group cg of 64 * NTW output columns).  Its
// 256 threads merge the records of (h, mb) exactly as attn_combine_kernel does and
// quantise the 16 x 128 head output into that head's packed operand tiles in LDS; its 4
// waves then multiply them by the head's 128 rows of the O weight, NTW column tiles each
// (NTW chosen for about 256 workgroups), and
// write split h of the O projection's partial sums (split-K over heads: split j is head
// j).  Per column tile the k-steps of the head are separate MFMAs added in k-step order,
// as the O GEMM with one split per head adds its waves' sums, so the partials are
// bitwise those of the merge kernel followed by that GEMM.  The weight loads are issued
// first and overlap the record loads.
template <int DT, int CH, int NTW, bool EXACT = false>
__global__ void __launch_bounds__(256) attn_merge_oproj_kernel(const AttnParams p, const GemmParams g, int nch) {
  constexpr int ADT = act_dtype_of(DT);
  constexpr int TBW = tile_bytes_of(DT), TBA = tile_bytes_of(ADT);
  constexpr int KPH = HD / kstep_of(DT);  // k-steps per head: 4 (bf16) or 1 (e4m3, MXFP4)
  __shared__ __attribute__((aligned(16))) uint8_t opnd[KPH * TBA];
  const int h = blockIdx.x, mb = blockIdx.y, cg = blockIdx.z, MB = p.MB;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pt0 = 4 * NTW * cg + NTW * wave;   // first column tile of this wave
  // the operand's static scale, requested first (after the merge it would cost a round trip)
  const float os = load_scale(p.out_scale_ptr, p.out_scale);

  Frag<DT> wf[NTW][KPH];
#pragma unroll
  for (int t = 0; t < NTW; ++t)
#pragma unroll
    for (int kk = 0; kk < KPH; ++kk)
      load_frag<DT, true>(wf[t][kk], g.w + ((size_t)(pt0 + t) * g.ksteps + h * KPH + kk) * TBW, lane);
  __builtin_amdgcn_sched_barrier(0);  // the weight loads go out first
  // Then every kernel argument that addresses the records, in one batch of scalar loads
  // (the empty asm only makes these values live here).  Read where the merge first uses
  // them, they came in two dependent scalar round trips ahead of the record loads (their
  // cache lines hold nothing the weight loads use; MB came from gridDim.y, an implicit
  // argument on a line of its own).  Measured on MI355X (paired, bitwise equal outputs,
  // with the Q/K/V scatter's arguments in the QKV GEMM): -0.08 / -0.25 us per layer
  // (bf16, M=50 / 10), -0.03 / -0.20 (e4m3), -0.13 / -0.23 (MXFP4 weights).  Requested at
  // kernel start instead, in the weights' batch: the same within 0.04 us.
  {
    const int pm = p.M, pnh = p.n_heads;
    const float* pws = p.workspace;
    asm volatile("" ::"s"(pm), "s"(pnh), "s"(pws), "s"(nch), "s"(MB));
  }

  const int tq = threadIdx.x >> 4;
  const int d0 = (threadIdx.x & 15) * 8;
  float o[8];
  merge_records<CH>(p, h, mb, MB, nch, tq, d0, mb * 16 + tq < p.M, o);
  const int m = mb * 16 + tq;
  store_operand4(opnd, ADT, 1, tq, d0, o[0], o[1], o[2], o[3], os, m >= p.M);
  store_operand4(opnd, ADT, 1, tq, d0 + 4, o[4], o[5], o[6], o[7], os, m >= p.M);
  if (m < p.M) {
    record_amax(p.amax, o[0], o[1], o[2], o[3]);
    record_amax(p.amax, o[4], o[5], o[6], o[7]);
  }
  __syncthreads();

  Frag<ADT> af[KPH];
#pragma unroll
  for (int kk = 0; kk < KPH; ++kk) load_frag<ADT, false>(af[kk], opnd + kk * TBA, lane);
  // The sums go straight from the MFMAs to memory through a buffer resource over this
  // head's partial slice; lanes of padding rows address past its end, where the hardware
  // drops the write.  No row-masked branch, which the MFMAs (they ignore EXEC) could be
  // sunk into, and no pass through LDS and a barrier to prevent that: measured on MI355X
  // (paired, bitwise equal outputs) -0.17 us/layer at M=50 in bf16, e4m3 and MXFP4, -0.1
  // at M=10.
  const int mrow = mb * 16 + (lane & 15);
  const unsigned slice = (unsigned)(g.M * g.N * 4);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(g.partials + (size_t)h * g.M * g.N), (short)0, (int)slice, kBufferWord3);
  const bool live = mrow < g.M;
  const unsigned rowoff = (unsigned)(mrow * g.N * 4);
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    f32x4 acc[KPH];
#pragma unroll
    for (int kk = 0; kk < KPH; ++kk) acc[kk] = mma_sel<EXACT>(wf[t][kk], af[kk], f32x4{0.f, 0.f, 0.f, 0.f});
    f32x4 v = acc[0];
#pragma unroll
    for (int kk = 1; kk < KPH; ++kk) v += acc[kk];
    const unsigned n0 = (unsigned)((pt0 + t) * 16 + 4 * (lane >> 4));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, (int)(live ? rowoff + 4 * n0 : slice), 0, 0);
  }
}

template <int NW, bool MULTI, bool REC>
static void launch_chunk(const AttnParams& p, dim3 g, hipStream_t s) {
  if (REC) hipLaunchKernelGGL((attn_chunk_kernel<NW, MULTI, true, FRT_BF16>), g, dim3(64 * NW), 0, s, p);
  else if (p.out_dtype == FRT_BF16) hipLaunchKernelGGL((attn_chunk_kernel<NW, MULTI, false, FRT_BF16>), g, dim3(64 * NW), 0, s, p);
  else hipLaunchKernelGGL((attn_chunk_kernel<NW, MULTI, false, FRT_E4M3>), g, dim3(64 * NW), 0, s, p);
}

template <int CH>
static void launch_combine(const AttnParams& p, int nch, hipStream_t s) {
  const dim3 g(p.n_heads, p.MB), b(256);
  if (p.out_dtype == FRT_BF16) hipLaunchKernelGGL((attn_combine_kernel<CH, FRT_BF16>), g, b, 0, s, p, nch);
  else hipLaunchKernelGGL((attn_combine_kernel<CH, FRT_E4M3>), g, b, 0, s, p, nch);
}

hipError_t launch_attention(const AttnParams& p_in, hipStream_t s) {
  AttnParams p = p_in;
  p.chunk_keys = attention_chunk_keys(p.M, p.n_heads, p.kv_len);
  const int nch = (p.kv_len + p.chunk_keys - 1) / p.chunk_keys;
  const dim3 g(p.n_heads, p.MB, nch);
  const bool rec = nch > 1;
  if (p.chunk_keys <= 64) rec ? launch_chunk<2, false, true>(p, g, s) : launch_chunk<2, false, false>(p, g, s);
  else if (p.chunk_keys <= 128) rec ? launch_chunk<4, false, true>(p, g, s) : launch_chunk<4, false, false>(p, g, s);
  else if (p.chunk_keys <= 256) rec ? launch_chunk<8, false, true>(p, g, s) : launch_chunk<8, false, false>(p, g, s);
  else rec ? launch_chunk<8, true, true>(p, g, s) : launch_chunk<8, true, false>(p, g, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !rec) return e;
  if (nch <= 8) launch_combine<8>(p, nch, s);
  else if (nch <= 16) launch_combine<16>(p, nch, s);
  else launch_combine<0>(p, nch, s);
  return hipGetLastError();
}

// Key chunks with partial records, then the merge fused with the O projection (`g` is the
// O GEMM's parameters with one split per head; the caller checks attention_oproj_fusable).
hipError_t launch_attention_oproj(const AttnParams& p_in, const GemmParams& g, hipStream_t s) {
  AttnParams p = p_in;
  p.chunk_keys = attention_chunk_keys(p.M, p.n_heads, p.kv_len);
  const int nch = (p.kv_len + p.chunk_keys - 1) / p.chunk_keys;
  const dim3 gc(p.n_heads, p.MB, nch);
  if (p.chunk_keys <= 64) launch_chunk<2, false, true>(p, gc, s);
  else launch_chunk<4, false, true>(p, gc, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // column tiles per wave: the widest that still gives 256 workgroups (measured at M=50:
  // 31.8 us/layer, against 32.6 with 128 workgroups and 32.2 with 512), else one
  const int base = p.n_heads * p.MB * (g.N / 256);
  const int ntw = base >= 256 ? 4 : (2 * base >= 256 ? 2 : 1);
  const dim3 gm(p.n_heads, p.MB, g.N / (64 * ntw)), b(256);
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, gm, b, 0, s, p, g, nch); };
  auto by_ntw = [&](auto k1, auto k2, auto k4) { ntw == 4 ? go(k4) : (ntw == 2 ? go(k2) : go(k1)); };
  // record slots per thread: the exact chunk count (a slot past the last chunk still
  // costs its loads; measured on MI355X, paired, bitwise equal outputs: 8 slots for the 7
  // chunks of M=50 cost 0.18 us per layer, 16 slots for the 13 chunks of M=10 0.33 us in
  // bf16 and 0.30 in e4m3)
  // e4m3 x e4m3 products exact at M <= 16, as in the O GEMM (the two stay bitwise equal)
#define FRT_MERGE_OPROJ(DT, CH, X)                                                                    \
  by_ntw(attn_merge_oproj_kernel<DT, CH, 1, X>, attn_merge_oproj_kernel<DT, CH, 2, X>, \
         attn_merge_oproj_kernel<DT, CH, 4, X>)
#define FRT_MERGE_OPROJ_DT(DT, X)                      \
  switch (nch) {                                       \
    case 2: FRT_MERGE_OPROJ(DT, 2, X); break;          \
    case 3: FRT_MERGE_OPROJ(DT, 3, X); break;          \
    case 4: FRT_MERGE_OPROJ(DT, 4, X); break;          \
    case 5: FRT_MERGE_OPROJ(DT, 5, X); break;          \
    case 6: FRT_MERGE_OPROJ(DT, 6, X); break;          \
    case 7: FRT_MERGE_OPROJ(DT, 7, X); break;          \
    case 8: FRT_MERGE_OPROJ(DT, 8, X); break;          \
    case 9: FRT_MERGE_OPROJ(DT, 9, X); break;          \
    case 10: FRT_MERGE_OPROJ(DT, 10, X); break;          \
    case 11: FRT_MERGE_OPROJ(DT, 11, X); break;          \
    case 12: FRT_MERGE_OPROJ(DT, 12, X); break;          \
    case 13: FRT_MERGE_OPROJ(DT, 13, X); break;          \
    case 14: FRT_MERGE_OPROJ(DT, 14, X); break;          \
    case 15: FRT_MERGE_OPROJ(DT, 15, X); break;          \
    default: FRT_MERGE_OPROJ(DT, 16, X); break;        \
  }
  switch (g.ab_dtype) {
    case FRT_BF16: FRT_MERGE_OPROJ_DT(FRT_BF16, false); break;
    case FRT_E4M3:
      if (e4m3_exact(g.M)) {
        FRT_MERGE_OPROJ_DT(FRT_E4M3, true);
      } else {
        FRT_MERGE_OPROJ_DT(FRT_E4M3, false);
      }
      break;
    default: FRT_MERGE_OPROJ_DT(FRT_MXFP4, false); break;
  }
#undef FRT_MERGE_OPROJ_DT
#undef FRT_MERGE_OPROJ
  return hipGetLastError();
}

// The fused pair applies when the key axis is cut into 2..16 chunks of at most 128 keys
// and the O projection's width is a multiple of 256.
bool attention_oproj_fusable(int M, int n_heads, int kv_len, int N) {
  const int ck = attention_chunk_keys(M, n_heads, kv_len), nch = (kv_len + ck - 1) / ck;
  return ck <= 128 && nch > 1 && nch <= 16 && N % 256 == 0;
}

int attention_kernel_count(int M, int n_heads, int kv_len) {
  const int ck = attention_chunk_keys(M, n_heads, kv_len);
  return (kv_len + ck - 1) / ck > 1 ? 2 : 1;
}

}  // namespace frt

using namespace frt;

extern "C" size_t frt_attention_workspace_bytes(int M, int n_heads, int head_dim, int kv_len) {
  if (M < 1 || M > kMaxM || n_heads < 1 || n_heads > 16 || head_dim != HD || kv_len < M || kv_len > 8192 + kMaxM)
    return 0;
  return attention_workspace_bytes(M, n_heads, kv_len);
}

extern "C" int frt_attention_prefix(void* stream, int M, int n_heads, int head_dim, int kv_len, const uint16_t* q_dev,
                                    const uint16_t* k_dev, const uint16_t* v_t_dev, int ldv, int out_dtype,
                                    float out_act_scale, void* operand_out_dev, void* workspace_dev,
                                    size_t workspace_bytes) {
  FRT_CHECK(q_dev && k_dev && v_t_dev && operand_out_dev && workspace_dev, FRT_E_NULL);
  FRT_CHECK(M >= 1 && M <= kMaxM, FRT_E_SHAPE);
  FRT_CHECK(head_dim == HD, FRT_E_SHAPE);
  FRT_CHECK(n_heads >= 1 && n_heads <= 16, FRT_E_SHAPE);
  FRT_CHECK(kv_len >= M && kv_len <= 8192 + kMaxM, FRT_E_SHAPE);
  FRT_CHECK(ldv >= (kv_len + 31) / 32 * 32 && ldv % 32 == 0, FRT_E_SHAPE);
  FRT_CHECK(is_ab_dtype(out_dtype), FRT_E_DTYPE);
  if (out_dtype == FRT_E4M3) FRT_CHECK(out_act_scale > 0.f && out_act_scale < __builtin_huge_valf(), FRT_E_ARG);
  const void* ptrs[] = {q_dev, k_dev, v_t_dev, operand_out_dev, workspace_dev};
  for (const void* x : ptrs) FRT_CHECK(aligned16(x), FRT_E_ALIGN);
  const size_t need = attention_workspace_bytes(M, n_heads, kv_len);
  FRT_CHECK(workspace_bytes >= need, FRT_E_WORKSPACE);
  const size_t ob = frt_operand_bytes(out_dtype, M, n_heads * HD);
  const size_t qb = (size_t)M * n_heads * HD * 2, kb = (size_t)kv_len * HD * 2, vb = (size_t)HD * ldv * 2;
  const void* ins[] = {q_dev, k_dev, v_t_dev};
  const size_t inb[] = {qb, kb, vb};
  for (int i = 0; i < 3; ++i) {
    FRT_CHECK(!overlaps(operand_out_dev, ob, ins[i], inb[i]), FRT_E_ALIAS);
    FRT_CHECK(!overlaps(workspace_dev, need, ins[i], inb[i]), FRT_E_ALIAS);
  }
  FRT_CHECK(!overlaps(workspace_dev, need, operand_out_dev, ob), FRT_E_ALIAS);
  AttnParams p{};
  p.M = M; p.MB = m_blocks(M); p.n_heads = n_heads; p.kv_len = kv_len;
  p.q = q_dev; p.k = k_dev; p.vt = v_t_dev; p.ldv = ldv;
  p.out_dtype = out_dtype; p.out_scale = out_dtype == FRT_E4M3 ? out_act_scale : 1.f; p.out_scale_ptr = nullptr;
  p.operand = (uint8_t*)operand_out_dev; p.workspace = (float*)workspace_dev;
  FRT_HIP(launch_attention(p, (hipStream_t)stream));
  return FRT_OK;
}
