// Attention of the M action rows over a cached bf16 prefix, fed straight from the fused
// QKV GEMM's split-K partials and writing the packed operand of the O projection.
//
// This step is not on the pages; it links the QKV-merged GEMM (observation-age notes
// "思考探索：具身推理加速，先看动作执行时观测有多旧", section "CUDA Graph 与图化简分别省掉什么":
// three projections of one input become one wider GEMM) to the O projection, and it is the
// consumer that reduces the QKV GEMM's FP32 partials (same notes, section
// "小 M GEMM 要看并行度，也要看归约代价").
//
// One workgroup per (query head, 16-row block); its 4 waves take interleaved 32-key
// blocks of [prefix ; own rows] and keep an online softmax each, merged in wave order at
// the end.  Scores are bf16 x bf16 MFMAs (exact products, fp32 sums); the probabilities
// multiply V as three bf16 pieces (hi + mid + lo carry all 24 bits of the fp32 value), so
// the output is fp32-accurate before it is quantised.
#include "frt_internal.hpp"

namespace frt {

constexpr int HD = 128;
constexpr int VT_STRIDE = HD + 8;  // padded row of the per-wave V staging (bank spread)

__device__ __forceinline__ bf16x8 bf16x8_from(const uint32_t* w4) {
  u32x4 v = {w4[0], w4[1], w4[2], w4[3]};
  return __builtin_bit_cast(bf16x8, v);
}

__global__ void __launch_bounds__(256) attn_prefix_kernel(const AttnParams p) {
  const int h = blockIdx.x, mb = blockIdx.y;
  // wave index made provably uniform: MFMAs ignore EXEC, so the per-wave key-block guard
  // must compile to a scalar branch
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int M = p.M, P = p.prefix_len, T = P + M;
  const int nqkv = (p.n_heads + 2) * HD;

  __shared__ __attribute__((aligned(16))) uint16_t Qs[16][HD];
  __shared__ __attribute__((aligned(16))) uint16_t Ko[kMaxM][HD];
  __shared__ __attribute__((aligned(16))) uint16_t Vo[kMaxM][HD];
  __shared__ __attribute__((aligned(16))) union {
    uint16_t vt[4][32][VT_STRIDE];
    f32x4 comb[4][8][64];
  } U;
  __shared__ float cm[4][16], cl[4][16];

  // ---- reduce the QKV partials (ascending split), recover scales, round to bf16
  const float as = load_scale(p.act_scale_ptr, p.act_scale);
  const size_t sst = (size_t)M * nqkv;
  auto qkv4 = [&](int m, int col) {
    const float* src = p.qkv + (size_t)m * nqkv + col;
    f32x4 v = *reinterpret_cast<const f32x4*>(src);
    for (int j = 1; j < p.splits; ++j) v += *reinterpret_cast<const f32x4*>(src + j * sst);
    v *= as;
    if (p.colscale) v *= *reinterpret_cast<const f32x4*>(p.colscale + col);
    u32x2 b;
    b.x = bf16_pack2(v.x, v.y);
    b.y = bf16_pack2(v.z, v.w);
    return b;
  };
  for (int i = threadIdx.x; i < 16 * (HD / 4); i += 256) {
    const int q = i / (HD / 4), c = (i % (HD / 4)) * 4, m = mb * 16 + q;
    u32x2 b = {0u, 0u};
    if (m < M) {
      b = qkv4(m, h * HD + c);
      if (p.qkv_out) *reinterpret_cast<u32x2*>(p.qkv_out + (size_t)m * nqkv + h * HD + c) = b;
    }
    *reinterpret_cast<u32x2*>(&Qs[q][c]) = b;
  }
  const bool write_kv = p.qkv_out && h == 0 && mb == 0;
  for (int i = threadIdx.x; i < kMaxM * (HD / 4); i += 256) {
    const int r = i / (HD / 4), c = (i % (HD / 4)) * 4;
    u32x2 kb = {0u, 0u}, vb = {0u, 0u};
    if (r < M) {
      kb = qkv4(r, p.n_heads * HD + c);
      vb = qkv4(r, p.n_heads * HD + HD + c);
      if (write_kv) {
        *reinterpret_cast<u32x2*>(p.qkv_out + (size_t)r * nqkv + p.n_heads * HD + c) = kb;
        *reinterpret_cast<u32x2*>(p.qkv_out + (size_t)r * nqkv + p.n_heads * HD + HD + c) = vb;
      }
    }
    *reinterpret_cast<u32x2*>(&Ko[r][c]) = kb;
    *reinterpret_cast<u32x2*>(&Vo[r][c]) = vb;
  }
  __syncthreads();

  // Q^T fragments (MFMA B operand): lane owns query L%16, d = 32*dc + 8*(L/16) + [0, 8)
  bf16x8 qf[4];
#pragma unroll
  for (int dc = 0; dc < 4; ++dc)
    qf[dc] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&Qs[lane & 15][32 * dc + 8 * (lane >> 4)]));

  const float scale = 0.08838834764831845f;  // 1 / sqrt(128)
  const float NEG_INF = -__builtin_huge_valf();
  float m_run = NEG_INF, l_run = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nkb = (T + 31) / 32;
  const int iters = (nkb + 3) / 4;
  const int g4 = lane >> 4;
  for (int it = 0; it < iters; ++it) {
    const int kb = it * 4 + wave;
    const bool active = kb < nkb;
    const int t0 = kb * 32;
    if (active) {  // stage this wave's 32 V rows (prefix from HBM, own rows from LDS)
      for (int i = lane; i < 32 * (HD / 8); i += 64) {
        const int r = i / (HD / 8), c = (i % (HD / 8)) * 8, t = t0 + r;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (t < P) v = *reinterpret_cast<const u32x4*>(p.v_prefix + (size_t)t * HD + c);
        else if (t < T) v = *reinterpret_cast<const u32x4*>(&Vo[t - P][c]);
        *reinterpret_cast<u32x4*>(&U.vt[wave][r][c]) = v;
      }
    }
    __syncthreads();
    if (active) {
      // S^T = K Q^T for keys t0 + 16*hf + [0,16): MFMA A operand = K rows
      f32x4 s[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        s[hf] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int t = t0 + 16 * hf + (lane & 15);
#pragma unroll
        for (int dc = 0; dc < 4; ++dc) {
          const int d0 = 32 * dc + 8 * g4;
          u32x4 kv = {0u, 0u, 0u, 0u};
          if (t < P) kv = *reinterpret_cast<const u32x4*>(p.k_prefix + (size_t)t * HD + d0);
          else if (t < T) kv = *reinterpret_cast<const u32x4*>(&Ko[t - P][d0]);
          s[hf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kv), qf[dc], s[hf], 0, 0, 0);
        }
      }
      // s[hf][r] = score of key t0 + 16*hf + 4*(L/16) + r for query L%16
      float bmax = NEG_INF;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = t0 + 16 * hf + 4 * g4 + r;
          s[hf][r] = t < T ? s[hf][r] * scale : NEG_INF;
          bmax = fmaxf(bmax, s[hf][r]);
        }
      bmax = fmaxf(bmax, __shfl_xor(bmax, 16, 64));
      bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
      const float m_new = fmaxf(m_run, bmax);
      const float alpha = expf(m_run - m_new);
      float pr[8];
      float psum = 0.f;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = expf(s[hf][r] - m_new);
          pr[4 * hf + r] = e;
          psum += e;
        }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      // P^T (MFMA B operand) in three bf16 pieces; slot j <-> key 4*(L/16)+j (j<4),
      // 16 + 4*(L/16) + j-4 (j>=4) of this 32-key block
      uint32_t hi[4], mid[4], lo[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float a0 = pr[2 * j], a1 = pr[2 * j + 1];
        const uint32_t h0 = bf16_bits(a0), h1 = bf16_bits(a1);
        a0 -= bf16_to_f32(h0);
        a1 -= bf16_to_f32(h1);
        const uint32_t m0 = bf16_bits(a0), m1 = bf16_bits(a1);
        a0 -= bf16_to_f32(m0);
        a1 -= bf16_to_f32(m1);
        hi[j] = h0 | (h1 << 16);
        mid[j] = m0 | (m1 << 16);
        lo[j] = bf16_bits(a0) | (bf16_bits(a1) << 16);
      }
      const bf16x8 phi = bf16x8_from(hi), pmid = bf16x8_from(mid), plo = bf16x8_from(lo);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        o[dt] *= alpha;
        const int d = 16 * dt + (lane & 15);
        uint32_t vw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int k0 = (2 * j < 4) ? 4 * g4 + 2 * j : 16 + 4 * g4 + 2 * j - 4;
          vw[j] = (uint32_t)U.vt[wave][k0][d] | ((uint32_t)U.vt[wave][k0 + 1][d] << 16);
        }
        const bf16x8 vf = bf16x8_from(vw);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, phi, o[dt], 0, 0, 0);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pmid, o[dt], 0, 0, 0);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, plo, o[dt], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // ---- merge the 4 waves' running softmax states in wave order
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (lane < 16) {
    cm[wave][lane] = m_run;
    cl[wave][lane] = l_run;
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) U.comb[wave][dt][lane] = o[dt];
  __syncthreads();

  const float os = load_scale(p.out_scale_ptr, p.out_scale);
  const int q = lane & 15;
  const int m = mb * 16 + q;
  float mx = NEG_INF;
  for (int w = 0; w < 4; ++w) mx = fmaxf(mx, cm[w][q]);
  float wgt[4], den = 0.f;
  for (int w = 0; w < 4; ++w) {
    wgt[w] = cm[w][q] == NEG_INF ? 0.f : expf(cm[w][q] - mx);
    den += wgt[w] * cl[w][q];
  }
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) {
    const int dt = 2 * wave + k2;
    f32x4 num = U.comb[0][dt][lane] * wgt[0];
    for (int w = 1; w < 4; ++w) num += U.comb[w][dt][lane] * wgt[w];
    const f32x4 ov = num / den;
    const int k = h * HD + 16 * dt + 4 * g4;
    store_operand4(p.operand, p.out_dtype, p.MB, m, k, ov.x, ov.y, ov.z, ov.w, os, m >= M);
  }
}

hipError_t launch_attention(const AttnParams& p, hipStream_t s) {
  hipLaunchKernelGGL(attn_prefix_kernel, dim3(p.n_heads, p.MB), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace frt

using namespace frt;

extern "C" int frt_attention_prefix(void* stream, int M, int n_heads, int head_dim, int prefix_len,
                                    const float* qkv_partials_dev, int qkv_splits, float qkv_act_scale,
                                    const float* qkv_colscale_dev, const uint16_t* k_prefix_dev,
                                    const uint16_t* v_prefix_dev, int out_dtype, float out_act_scale,
                                    void* operand_out_dev, uint16_t* qkv_out_dev) {
  FRT_CHECK(qkv_partials_dev && operand_out_dev, FRT_E_NULL);
  FRT_CHECK(prefix_len == 0 || (k_prefix_dev && v_prefix_dev), FRT_E_NULL);
  FRT_CHECK(M >= 1 && M <= kMaxM, FRT_E_SHAPE);
  FRT_CHECK(head_dim == HD, FRT_E_SHAPE);
  FRT_CHECK(n_heads >= 1 && n_heads <= 16, FRT_E_SHAPE);
  FRT_CHECK(prefix_len >= 0 && prefix_len <= 8192, FRT_E_SHAPE);
  FRT_CHECK(qkv_splits >= 1 && qkv_splits <= kMaxSplits, FRT_E_SPLITK);
  FRT_CHECK(is_ab_dtype(out_dtype), FRT_E_DTYPE);
  FRT_CHECK(qkv_act_scale > 0.f && qkv_act_scale < __builtin_huge_valf(), FRT_E_ARG);
  if (out_dtype == FRT_E4M3) FRT_CHECK(out_act_scale > 0.f && out_act_scale < __builtin_huge_valf(), FRT_E_ARG);
  const void* ptrs[] = {qkv_partials_dev, qkv_colscale_dev, k_prefix_dev, v_prefix_dev, operand_out_dev,
                        qkv_out_dev};
  for (const void* q : ptrs) FRT_CHECK(aligned16(q), FRT_E_ALIGN);
  const size_t nqkv = (size_t)(n_heads + 2) * HD;
  const size_t ob = frt_operand_bytes(out_dtype, M, n_heads * HD);
  const size_t pb = (size_t)qkv_splits * M * nqkv * 4;
  FRT_CHECK(!overlaps(operand_out_dev, ob, qkv_partials_dev, pb), FRT_E_ALIAS);
  FRT_CHECK(!overlaps(qkv_out_dev, (size_t)M * nqkv * 2, qkv_partials_dev, pb), FRT_E_ALIAS);
  FRT_CHECK(!overlaps(qkv_out_dev, (size_t)M * nqkv * 2, operand_out_dev, ob), FRT_E_ALIAS);
  AttnParams p{};
  p.M = M; p.MB = m_blocks(M); p.n_heads = n_heads; p.prefix_len = prefix_len;
  p.qkv = qkv_partials_dev; p.splits = qkv_splits; p.act_scale = qkv_act_scale; p.act_scale_ptr = nullptr;
  p.colscale = qkv_colscale_dev; p.k_prefix = k_prefix_dev; p.v_prefix = v_prefix_dev;
  p.out_dtype = out_dtype; p.out_scale = out_dtype == FRT_E4M3 ? out_act_scale : 1.f; p.out_scale_ptr = nullptr;
  p.operand = (uint8_t*)operand_out_dev; p.qkv_out = qkv_out_dev;
  FRT_HIP(launch_attention(p, (hipStream_t)stream));
  return FRT_OK;
}
