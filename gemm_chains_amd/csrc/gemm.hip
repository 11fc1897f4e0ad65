// Skinny split-K GEMM on CDNA4 MFMA, and the split-K consumer.
//
// Pages: observation-age notes ("思考探索：具身推理加速，先看动作执行时观测有多旧"),
// section "小 M GEMM 要看并行度，也要看归约代价": C = A W with few rows (M = 10 or 50 action
// rows), cut along K into s partial products C = sum_j A_j W_j held in FP32 and reduced
// by the next consumer, which also continues the transformation it needs; the path keeps
// re-laid-out weight copies.  Section "静态量化改变了两次矩阵乘之间的工作": the GEMM's scale
// recovery remains after static quantisation (applied here after the fixed-order sum).
//
// Mapping (gfx950): the weight tile is the MFMA's A operand (16 output columns x one
// k-step) and the activation tile its B operand (one k-step x 16 action rows), so the
// 16x16 accumulator holds C^T for 16 columns x 16 rows and M (<= 64) occupies 1..4
// column blocks.  Weights are pre-packed so that one 16-byte load per lane is one tile
// (1 KB per wave load, fully coalesced, straight into VGPRs with no LDS round trip);
// activations come packed the same way from the producer.  A workgroup owns NT column
// tiles and one K-chunk; its waves split the chunk's k-steps and are summed through LDS
// in wave order, so every result is bitwise deterministic.
#include "frt_internal.hpp"

namespace frt {

template <int DT>
struct Frag;
template <>
struct Frag<FRT_BF16> {
  u32x4 v;
};
template <>
struct Frag<FRT_E4M3> {
  u32x4 v0, v1;
};

template <int DT>
__device__ __forceinline__ void load_frag(Frag<DT>& f, const uint8_t* tile, int lane, bool stream);
template <>
__device__ __forceinline__ void load_frag<FRT_BF16>(Frag<FRT_BF16>& f, const uint8_t* tile, int lane,
                                                    bool stream) {
  const u32x4* p = reinterpret_cast<const u32x4*>(tile + lane * 16);
  f.v = stream ? __builtin_nontemporal_load(p) : *p;
}
template <>
__device__ __forceinline__ void load_frag<FRT_E4M3>(Frag<FRT_E4M3>& f, const uint8_t* tile, int lane,
                                                    bool stream) {
  const u32x4* p0 = reinterpret_cast<const u32x4*>(tile + lane * 16);
  const u32x4* p1 = reinterpret_cast<const u32x4*>(tile + 1024 + lane * 16);
  if (stream) {
    f.v0 = __builtin_nontemporal_load(p0);
    f.v1 = __builtin_nontemporal_load(p1);
  } else {
    f.v0 = *p0;
    f.v1 = *p1;
  }
}

__device__ __forceinline__ f32x4 mma(const Frag<FRT_BF16>& w, const Frag<FRT_BF16>& a, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w.v),
                                                 __builtin_bit_cast(bf16x8, a.v), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const Frag<FRT_E4M3>& w, const Frag<FRT_E4M3>& a, f32x4 c) {
  i32x8 wa, aa;
  wa[0] = (int)w.v0.x; wa[1] = (int)w.v0.y; wa[2] = (int)w.v0.z; wa[3] = (int)w.v0.w;
  wa[4] = (int)w.v1.x; wa[5] = (int)w.v1.y; wa[6] = (int)w.v1.z; wa[7] = (int)w.v1.w;
  aa[0] = (int)a.v0.x; aa[1] = (int)a.v0.y; aa[2] = (int)a.v0.z; aa[3] = (int)a.v0.w;
  aa[4] = (int)a.v1.x; aa[5] = (int)a.v1.y; aa[6] = (int)a.v1.z; aa[7] = (int)a.v1.w;
  // format 0/0 = OCP e4m3 for both operands; E8M0 block scales 127 = 2^0 (unscaled)
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wa, aa, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

// Epilogue for one 16x16 accumulator fragment when the whole K was summed in this kernel.
// v[r] = C^T[n0 + r][m] for lane-owned (m, n0..n0+3).
__device__ __forceinline__ void store_c4(const GemmParams& p, int m, int n0, f32x4 v, float as) {
  if (m >= p.M) return;
  f32x4 c = v * as;
  if (p.colscale) c *= *reinterpret_cast<const f32x4*>(p.colscale + n0);
  if (p.epi == kEpiQkv) {
    store_qkv4(p.q_out, p.k_out, p.v_out, p.nq, p.hd, p.v_ld, m, n0, c);
  } else if (p.epi == FRT_EPI_STORE_F32) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + (size_t)m * p.N + n0) = c;
  } else {
    u32x2 w;
    w.x = bf16_pack2(c.x, c.y);
    w.y = bf16_pack2(c.z, c.w);
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.out) + (size_t)m * p.N + n0) = w;
  }
}

template <int DT, int MB, int NT>
__global__ void __launch_bounds__(512) skinny_gemm_kernel(const GemmParams p) {
  constexpr int TB = DT == FRT_BF16 ? 1024 : 2048;
  // k-steps per pipeline stage: two stages of (NT + MB) fragments plus the accumulators
  // should stay within ~160 VGPRs so that two waves fit per SIMD without spills
  constexpr int NV = DT == FRT_BF16 ? 1 : 2;
  constexpr int U_fit = (160 - 4 * NT * MB) / (2 * (NT + MB) * 4 * NV);
  constexpr int U = U_fit < 1 ? 1 : (U_fit > 4 ? 4 : U_fit);
  extern __shared__ f32x4 red[];  // [kwaves][NT*MB][64]

  const int lane = threadIdx.x & 63;
  // wave index made provably uniform: MFMAs ignore EXEC, so every branch around them must
  // be a scalar branch, never an EXEC-masked one
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kw = p.kwaves;
  const int g = blockIdx.x;        // column-tile group: packed tiles [g*NT, g*NT + NT)
  const int split = blockIdx.y;
  const int KS = p.K / (DT == FRT_BF16 ? 32 : 128);
  const int per = p.ksteps_per_split / kw;
  const int ks_begin = split * p.ksteps_per_split + wave * per;
  const int ks_end = ks_begin + per;

  const uint8_t* wbase[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) wbase[t] = p.w + (size_t)(g * NT + t) * KS * TB;

  f32x4 acc[NT][MB];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int b = 0; b < MB; ++b) acc[t][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  Frag<DT> wf[2][U][NT];
  Frag<DT> af[2][U][MB];
  auto load_stage = [&](int buf, int ks0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ks = ks0 + u;
      if (ks < ks_end) {
#pragma unroll
        for (int t = 0; t < NT; ++t) load_frag<DT>(wf[buf][u][t], wbase[t] + (size_t)ks * TB, lane, true);
#pragma unroll
        for (int b = 0; b < MB; ++b)
          load_frag<DT>(af[buf][u][b], p.a + ((size_t)ks * MB + b) * TB, lane, false);
      }
    }
  };
  auto compute_stage = [&](int buf, int ks0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ks0 + u < ks_end) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int b = 0; b < MB; ++b) acc[t][b] = mma(wf[buf][u][t], af[buf][u][b], acc[t][b]);
      }
    }
  };

  // two-stage register pipeline: stage i+1's loads are in flight while stage i computes
  if (ks_begin < ks_end) load_stage(0, ks_begin);
  for (int ks0 = ks_begin; ks0 < ks_end; ks0 += 2 * U) {
    if (ks0 + U < ks_end) load_stage(1, ks0 + U);
    compute_stage(0, ks0);
    if (ks0 + U < ks_end) {
      if (ks0 + 2 * U < ks_end) load_stage(0, ks0 + 2 * U);
      compute_stage(1, ks0 + U);
    }
  }

  const float as = load_scale(p.act_scale_ptr, p.act_scale);
  const bool partial_out = (p.epi == FRT_EPI_NONE) || p.splits > 1;
  constexpr int NF = NT * MB;

  // combine the kw waves' sums in wave order (LDS), then each wave finishes some fragments
  if (kw > 1) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int b = 0; b < MB; ++b) red[((size_t)wave * NF + t * MB + b) * 64 + lane] = acc[t][b];
    __syncthreads();
  }

  auto finish = [&](int t, int b, f32x4 v) {
    const int lt = logical_tile_of(p.layout, p.N, g * NT + t);
    const int n0 = lt * 16 + 4 * (lane >> 4);
    const int m = b * 16 + (lane & 15);
    if (partial_out) {
      if (m < p.M) *reinterpret_cast<f32x4*>(p.partials + ((size_t)split * p.M + m) * p.N + n0) = v;
    } else {
      store_c4(p, m, n0, v, as);
    }
  };
  const float os = load_scale(p.out_scale_ptr, p.out_scale);
  // SiLU-gate epilogue: packed tiles 2i (gate) and 2i+1 (up) of this workgroup pair up
  auto finish_pair = [&](int tp, int b, f32x4 vg, f32x4 vu) {
    const int ng = logical_tile_of(p.layout, p.N, g * NT + 2 * tp) * 16 + 4 * (lane >> 4);
    const int nu = logical_tile_of(p.layout, p.N, g * NT + 2 * tp + 1) * 16 + 4 * (lane >> 4);
    const int m = b * 16 + (lane & 15);
    f32x4 cg = vg * as, cu = vu * as;
    if (p.colscale) {
      cg *= *reinterpret_cast<const f32x4*>(p.colscale + ng);
      cu *= *reinterpret_cast<const f32x4*>(p.colscale + nu);
    }
    float z[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) z[r] = silu_f(cg[r]) * cu[r];
    store_operand4(reinterpret_cast<uint8_t*>(p.out), p.out_dtype, MB, m, ng, z[0], z[1], z[2], z[3], os,
                   m >= p.M);
    if (m < p.M) record_amax(p.amax, z[0], z[1], z[2], z[3]);
  };
  const bool silu = !partial_out && p.epi == FRT_EPI_SILU_GATE_QUANT;

  if (kw == 1) {
    if (silu) {
#pragma unroll
      for (int tp = 0; tp < NT / 2; ++tp)
#pragma unroll
        for (int b = 0; b < MB; ++b) finish_pair(tp, b, acc[2 * tp][b], acc[2 * tp + 1][b]);
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int b = 0; b < MB; ++b) finish(t, b, acc[t][b]);
    }
    return;
  }
  auto sum_waves = [&](int f) {
    f32x4 v = red[(size_t)f * 64 + lane];
    for (int w2 = 1; w2 < kw; ++w2) v += red[((size_t)w2 * NF + f) * 64 + lane];
    return v;
  };
  if (silu) {
    constexpr int NPAIR = (NT / 2) * MB;
    for (int f = wave; f < NPAIR; f += kw) {
      const int tp = f / MB, b = f % MB;
      finish_pair(tp, b, sum_waves((2 * tp) * MB + b), sum_waves((2 * tp + 1) * MB + b));
    }
  } else {
    for (int f = wave; f < NF; f += kw) finish(f / MB, f % MB, sum_waves(f));
  }
}

// Consumer: fixed-order split-K reduction + scale recovery + epilogue.  One thread per
// 4 consecutive columns of one row (rows up to Mp for the SiLU epilogue, whose padding
// rows are written as zero codes).  SPL >= splits is a compile-time bound so that every
// slice's load is issued before the sum starts (one memory latency, not one per slice).
template <int SPL>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const ReduceParams p) {
  const float as = load_scale(p.act_scale_ptr, p.act_scale);
  const int ncols = p.epi == FRT_EPI_SILU_GATE_QUANT ? p.N / 2 : p.N;
  const int q4 = ncols / 4;
  const int rows = p.epi == FRT_EPI_SILU_GATE_QUANT ? p.MB * 16 : p.M;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * q4) return;
  const int m = idx / q4;
  const int n0 = (idx % q4) * 4;
  const size_t sstride = (size_t)p.M * p.N;
  auto reduce4 = [&](int n) {
    const float* src = p.partials + (size_t)m * p.N + n;
    f32x4 pj[SPL];
#pragma unroll
    for (int j = 0; j < SPL; ++j)
      if (j < p.splits) pj[j] = *reinterpret_cast<const f32x4*>(src + j * sstride);
    f32x4 v = pj[0];
#pragma unroll
    for (int j = 1; j < SPL; ++j)
      if (j < p.splits) v += pj[j];
    v *= as;
    if (p.colscale) v *= *reinterpret_cast<const f32x4*>(p.colscale + n);
    return v;
  };
  if (p.epi == FRT_EPI_SILU_GATE_QUANT) {
    const float os = load_scale(p.out_scale_ptr, p.out_scale);
    if (m >= p.M) {
      store_operand4(reinterpret_cast<uint8_t*>(p.out), p.out_dtype, p.MB, m, n0, 0.f, 0.f, 0.f, 0.f, os, true);
      return;
    }
    const f32x4 cg = reduce4(n0), cu = reduce4(p.N / 2 + n0);
    float z[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) z[r] = silu_f(cg[r]) * cu[r];
    store_operand4(reinterpret_cast<uint8_t*>(p.out), p.out_dtype, p.MB, m, n0, z[0], z[1], z[2], z[3], os, false);
    record_amax(p.amax, z[0], z[1], z[2], z[3]);
    return;
  }
  const f32x4 c = reduce4(n0);
  if (p.epi == kEpiQkv) {
    store_qkv4(p.q_out, p.k_out, p.v_out, p.nq, p.hd, p.v_ld, m, n0, c);
  } else if (p.epi == FRT_EPI_STORE_F32) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + (size_t)m * p.N + n0) = c;
  } else {
    u32x2 w;
    w.x = bf16_pack2(c.x, c.y);
    w.y = bf16_pack2(c.z, c.w);
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.out) + (size_t)m * p.N + n0) = w;
  }
}

// ------------------------------------------------------------------ launch plumbing
template <int DT, int MB, int NT>
static hipError_t launch_t(const GemmParams& p, hipStream_t s) {
  const int groups = p.N / 16 / NT;
  const size_t lds = p.kwaves > 1 ? (size_t)p.kwaves * NT * MB * 64 * sizeof(f32x4) : 0;
  hipLaunchKernelGGL((skinny_gemm_kernel<DT, MB, NT>), dim3(groups, p.splits), dim3(64 * p.kwaves), lds, s, p);
  return hipGetLastError();
}

template <int DT, int MB>
static hipError_t launch_nt(const GemmParams& p, int nt, hipStream_t s) {
  switch (nt) {
    case 1: return launch_t<DT, MB, 1>(p, s);
    case 2: return launch_t<DT, MB, 2>(p, s);
    default: return launch_t<DT, MB, 4>(p, s);
  }
}

template <int DT>
static hipError_t launch_mb(const GemmParams& p, int nt, hipStream_t s) {
  switch (p.MB) {
    case 1: return launch_nt<DT, 1>(p, nt, s);
    case 2: return launch_nt<DT, 2>(p, nt, s);
    case 3: return launch_nt<DT, 3>(p, nt, s);
    default: return launch_nt<DT, 4>(p, nt, s);
  }
}

// Column tiles per workgroup: the SiLU epilogue needs gate/up pairs (even NT); otherwise
// pick the widest tile group that still leaves >= 256 workgroups (one per CU).
static int choose_nt(const GemmParams& p) {
  const int tiles = p.N / 16;
  const bool pairs = p.splits == 1 && p.epi == FRT_EPI_SILU_GATE_QUANT;
  int nt = pairs ? 2 : 1;
  for (int cand : {4, 2}) {
    if (tiles % cand) continue;
    if (pairs && cand % 2) continue;
    if ((tiles / cand) * p.splits >= 256) { nt = cand > nt ? cand : nt; break; }
  }
  if (tiles % nt) nt = 1;
  return nt;
}

// Waves per workgroup splitting a K-chunk: up to 8, dividing the chunk's k-steps, and
// keeping the cross-wave LDS buffer (kw * frags * 1 KB) within 64 KB.
int choose_kwaves(int ksteps_per_split, int frags) {
  int kw = 1;
  while (kw < 8 && ksteps_per_split % (kw * 2) == 0 && (kw * 2) * frags <= 64) kw *= 2;
  return kw;
}

hipError_t launch_gemm(const GemmParams& p_in, hipStream_t s) {
  GemmParams p = p_in;
  const int nt = choose_nt(p);
  p.kwaves = choose_kwaves(p.ksteps_per_split, nt * p.MB);
  return p.ab_dtype == FRT_BF16 ? launch_mb<FRT_BF16>(p, nt, s) : launch_mb<FRT_E4M3>(p, nt, s);
}

hipError_t launch_reduce(const ReduceParams& p, hipStream_t s) {
  const int ncols = p.epi == FRT_EPI_SILU_GATE_QUANT ? p.N / 2 : p.N;
  const int rows = p.epi == FRT_EPI_SILU_GATE_QUANT ? p.MB * 16 : p.M;
  const int total = rows * (ncols / 4);
  const dim3 g((total + 255) / 256), b(256);
  if (p.splits <= 2) hipLaunchKernelGGL(splitk_reduce_kernel<2>, g, b, 0, s, p);
  else if (p.splits <= 4) hipLaunchKernelGGL(splitk_reduce_kernel<4>, g, b, 0, s, p);
  else if (p.splits <= 8) hipLaunchKernelGGL(splitk_reduce_kernel<8>, g, b, 0, s, p);
  else hipLaunchKernelGGL(splitk_reduce_kernel<16>, g, b, 0, s, p);
  return hipGetLastError();
}

// Split-K choice (measured on MI355X at the action-decoder shapes).  When the GEMM ends
// in an epilogue, s > 1 costs a separate consumer kernel (~1.6 us of graph dispatch plus
// its own memory round trip), more than the extra parallelism buys: s = 1.  When the
// partials are the output (the next producer reduces them anyway), split until there are
// two workgroups per CU (512) while every chunk keeps at least 4 k-steps.
int choose_splits(int M, int N, int K, int dtype, int epi) {
  (void)M;
  if (epi != FRT_EPI_NONE) return 1;
  const int tiles = N / 16;
  const int ksteps = K / kstep_of(dtype);
  int s = 1;
  while (s < 16 && tiles * s < 512 && ksteps % (2 * s) == 0 && ksteps / (2 * s) >= 4) s *= 2;
  return s;
}

}  // namespace frt

using namespace frt;

static int validate_epilogue_out(int M, int N, int epi, const void* out_dev, int out_dtype, float out_act_scale) {
  if (epi == FRT_EPI_NONE) return FRT_OK;
  FRT_CHECK(epi == FRT_EPI_STORE_F32 || epi == FRT_EPI_STORE_BF16 || epi == FRT_EPI_SILU_GATE_QUANT, FRT_E_ARG);
  FRT_CHECK(out_dev, FRT_E_NULL);
  FRT_CHECK(aligned16(out_dev), FRT_E_ALIGN);
  if (epi == FRT_EPI_SILU_GATE_QUANT) {
    FRT_CHECK(is_ab_dtype(out_dtype), FRT_E_DTYPE);
    FRT_CHECK(N % 32 == 0 && (N / 2) % kstep_of(out_dtype) == 0, FRT_E_SHAPE);
    if (out_dtype == FRT_E4M3) FRT_CHECK(out_act_scale > 0.f && out_act_scale < __builtin_huge_valf(), FRT_E_ARG);
  }
  (void)M;
  return FRT_OK;
}

static size_t epilogue_out_bytes(int M, int N, int epi, int out_dtype) {
  switch (epi) {
    case FRT_EPI_STORE_F32: return (size_t)M * N * 4;
    case FRT_EPI_STORE_BF16: return (size_t)M * N * 2;
    case FRT_EPI_SILU_GATE_QUANT: return frt_operand_bytes(out_dtype, M, N / 2);
    default: return 0;
  }
}

extern "C" int frt_splitk_choose(int M, int N, int K, int ab_dtype) {
  if (M < 1 || M > kMaxM || N < 16 || N % 16 || !is_ab_dtype(ab_dtype) || K < kstep_of(ab_dtype) ||
      K % kstep_of(ab_dtype))
    return 0;
  return choose_splits(M, N, K, ab_dtype, FRT_EPI_NONE);
}

extern "C" int frt_skinny_gemm_splitk(void* stream, int M, int N, int K, int splits, int ab_dtype,
                                      int layout, const void* a_packed_dev, const void* w_packed_dev,
                                      const float* w_colscale_dev, float act_scale, float* partials_dev,
                                      size_t partials_bytes, int epi, void* out_dev, int out_dtype,
                                      float out_act_scale) {
  FRT_CHECK(a_packed_dev && w_packed_dev, FRT_E_NULL);
  FRT_CHECK(is_ab_dtype(ab_dtype), FRT_E_DTYPE);
  FRT_CHECK(M >= 1 && M <= kMaxM, FRT_E_SHAPE);
  FRT_CHECK(N >= 16 && N % 16 == 0 && N <= (1 << 20), FRT_E_SHAPE);
  FRT_CHECK(K >= kstep_of(ab_dtype) && K % kstep_of(ab_dtype) == 0 && K <= (1 << 16), FRT_E_SHAPE);
  FRT_CHECK(layout == FRT_W_PLAIN || layout == FRT_W_GATE_UP, FRT_E_ARG);
  if (layout == FRT_W_GATE_UP) FRT_CHECK(N % 32 == 0, FRT_E_SHAPE);
  FRT_CHECK(act_scale > 0.f && act_scale < __builtin_huge_valf(), FRT_E_ARG);
  FRT_CHECK(epi >= FRT_EPI_NONE && epi <= FRT_EPI_SILU_GATE_QUANT, FRT_E_ARG);
  if (splits == 0) splits = choose_splits(M, N, K, ab_dtype, epi);
  FRT_CHECK(is_split(splits), FRT_E_SPLITK);
  const int ksteps = K / kstep_of(ab_dtype);
  FRT_CHECK(ksteps % splits == 0, FRT_E_SPLITK);
  FRT_CHECK(epi >= FRT_EPI_NONE && epi <= FRT_EPI_SILU_GATE_QUANT, FRT_E_ARG);
  if (epi == FRT_EPI_SILU_GATE_QUANT) FRT_CHECK(layout == FRT_W_GATE_UP || splits > 1, FRT_E_ARG);
  int st = validate_epilogue_out(M, N, epi, out_dev, out_dtype, out_act_scale);
  if (st != FRT_OK) return st;
  const void* ptrs[] = {a_packed_dev, w_packed_dev, w_colscale_dev, partials_dev};
  for (const void* q : ptrs) FRT_CHECK(aligned16(q), FRT_E_ALIGN);
  const bool need_partials = epi == FRT_EPI_NONE || splits > 1;
  const size_t pbytes = (size_t)splits * M * N * 4;
  if (need_partials) {
    FRT_CHECK(partials_dev, FRT_E_NULL);
    FRT_CHECK(partials_bytes >= pbytes, FRT_E_WORKSPACE);
  }
  const size_t ab = frt_operand_bytes(ab_dtype, M, K);
  const size_t wb = frt_weight_bytes(ab_dtype, K, N);
  const size_t ob = epilogue_out_bytes(M, N, epi, out_dtype);
  if (need_partials) {
    FRT_CHECK(!overlaps(partials_dev, pbytes, a_packed_dev, ab), FRT_E_ALIAS);
    FRT_CHECK(!overlaps(partials_dev, pbytes, w_packed_dev, wb), FRT_E_ALIAS);
    FRT_CHECK(!overlaps(partials_dev, pbytes, out_dev, ob), FRT_E_ALIAS);
  }
  FRT_CHECK(!overlaps(out_dev, ob, a_packed_dev, ab), FRT_E_ALIAS);
  FRT_CHECK(!overlaps(out_dev, ob, w_packed_dev, wb), FRT_E_ALIAS);

  GemmParams p{};
  p.M = M; p.N = N; p.K = K; p.MB = m_blocks(M); p.splits = splits;
  p.ab_dtype = ab_dtype; p.layout = layout; p.ksteps_per_split = ksteps / splits;
  p.a = (const uint8_t*)a_packed_dev; p.w = (const uint8_t*)w_packed_dev; p.colscale = w_colscale_dev;
  p.act_scale = act_scale; p.act_scale_ptr = nullptr; p.partials = partials_dev;
  p.epi = epi; p.out = out_dev; p.out_dtype = out_dtype; p.out_scale = out_dtype == FRT_E4M3 ? out_act_scale : 1.f;
  p.out_scale_ptr = nullptr;
  hipStream_t s = (hipStream_t)stream;
  FRT_HIP(launch_gemm(p, s));
  if (splits > 1 && epi != FRT_EPI_NONE) {
    ReduceParams r{};
    r.M = M; r.N = N; r.MB = p.MB; r.splits = splits; r.partials = partials_dev;
    r.act_scale = act_scale; r.act_scale_ptr = nullptr; r.colscale = w_colscale_dev; r.epi = epi;
    r.out = out_dev; r.out_dtype = out_dtype; r.out_scale = p.out_scale; r.out_scale_ptr = nullptr;
    FRT_HIP(launch_reduce(r, s));
  }
  return FRT_OK;
}

extern "C" int frt_splitk_reduce(void* stream, int M, int N, int splits, const float* partials_dev,
                                 float act_scale, const float* w_colscale_dev, int epi, void* out_dev,
                                 int out_dtype, float out_act_scale) {
  FRT_CHECK(partials_dev, FRT_E_NULL);
  FRT_CHECK(M >= 1 && M <= kMaxM, FRT_E_SHAPE);
  FRT_CHECK(N >= 16 && N % 16 == 0, FRT_E_SHAPE);
  FRT_CHECK(splits >= 1 && splits <= kMaxSplits, FRT_E_SPLITK);
  FRT_CHECK(epi == FRT_EPI_STORE_F32 || epi == FRT_EPI_STORE_BF16 || epi == FRT_EPI_SILU_GATE_QUANT, FRT_E_ARG);
  FRT_CHECK(act_scale > 0.f && act_scale < __builtin_huge_valf(), FRT_E_ARG);
  int st = validate_epilogue_out(M, N, epi, out_dev, out_dtype, out_act_scale);
  if (st != FRT_OK) return st;
  FRT_CHECK(aligned16(partials_dev) && aligned16(w_colscale_dev), FRT_E_ALIGN);
  const size_t pbytes = (size_t)splits * M * N * 4;
  FRT_CHECK(!overlaps(partials_dev, pbytes, out_dev, epilogue_out_bytes(M, N, epi, out_dtype)), FRT_E_ALIAS);
  ReduceParams r{};
  r.M = M; r.N = N; r.MB = m_blocks(M); r.splits = splits; r.partials = partials_dev;
  r.act_scale = act_scale; r.act_scale_ptr = nullptr; r.colscale = w_colscale_dev; r.epi = epi;
  r.out = out_dev; r.out_dtype = out_dtype; r.out_scale = out_dtype == FRT_E4M3 ? out_act_scale : 1.f;
  r.out_scale_ptr = nullptr;
  FRT_HIP(launch_reduce(r, (hipStream_t)stream));
  return FRT_OK;
}

extern "C" int frt_skinny_gemm_qkv(void* stream, int M, int K, int n_heads, int head_dim, int splits, int ab_dtype,
                                   const void* a_packed_dev, const void* w_packed_dev, const float* w_colscale_dev,
                                   float act_scale, float* partials_dev, size_t partials_bytes, uint16_t* q_out_dev,
                                   uint16_t* k_out_dev, uint16_t* v_t_out_dev, int v_ld) {
  uint16_t* v_out_dev = v_t_out_dev;
  FRT_CHECK(a_packed_dev && w_packed_dev && q_out_dev && k_out_dev && v_out_dev, FRT_E_NULL);
  FRT_CHECK(is_ab_dtype(ab_dtype), FRT_E_DTYPE);
  FRT_CHECK(M >= 1 && M <= kMaxM, FRT_E_SHAPE);
  FRT_CHECK(n_heads >= 1 && n_heads <= 64 && head_dim >= 16 && head_dim % 16 == 0, FRT_E_SHAPE);
  FRT_CHECK(v_ld >= M, FRT_E_SHAPE);
  const int N = (n_heads + 2) * head_dim;
  FRT_CHECK(K >= kstep_of(ab_dtype) && K % kstep_of(ab_dtype) == 0 && K <= (1 << 16), FRT_E_SHAPE);
  FRT_CHECK(act_scale > 0.f && act_scale < __builtin_huge_valf(), FRT_E_ARG);
  if (splits == 0) splits = choose_splits(M, N, K, ab_dtype, kEpiQkv);
  FRT_CHECK(is_split(splits), FRT_E_SPLITK);
  const int ksteps = K / kstep_of(ab_dtype);
  FRT_CHECK(ksteps % splits == 0, FRT_E_SPLITK);
  const void* ptrs[] = {a_packed_dev, w_packed_dev, w_colscale_dev, partials_dev, q_out_dev, k_out_dev};
  for (const void* q : ptrs) FRT_CHECK(aligned16(q), FRT_E_ALIGN);
  FRT_CHECK(((uintptr_t)v_out_dev & 1u) == 0, FRT_E_ALIGN);  // V^T is written element by element
  const size_t pbytes = (size_t)splits * M * N * 4;
  if (splits > 1) {
    FRT_CHECK(partials_dev, FRT_E_NULL);
    FRT_CHECK(partials_bytes >= pbytes, FRT_E_WORKSPACE);
  }
  const size_t ab = frt_operand_bytes(ab_dtype, M, K), wb = frt_weight_bytes(ab_dtype, K, N);
  const size_t qb = (size_t)M * n_heads * head_dim * 2, kb = (size_t)M * head_dim * 2;
  const size_t vb = ((size_t)(head_dim - 1) * v_ld + M) * 2;
  const void* outs[] = {q_out_dev, k_out_dev, v_out_dev};
  const size_t outb[] = {qb, kb, vb};
  for (int i = 0; i < 3; ++i) {
    FRT_CHECK(!overlaps(outs[i], outb[i], a_packed_dev, ab), FRT_E_ALIAS);
    FRT_CHECK(!overlaps(outs[i], outb[i], w_packed_dev, wb), FRT_E_ALIAS);
    if (splits > 1) FRT_CHECK(!overlaps(outs[i], outb[i], partials_dev, pbytes), FRT_E_ALIAS);
    for (int j = i + 1; j < 3; ++j) FRT_CHECK(!overlaps(outs[i], outb[i], outs[j], outb[j]), FRT_E_ALIAS);
  }
  if (splits > 1) {
    FRT_CHECK(!overlaps(partials_dev, pbytes, a_packed_dev, ab), FRT_E_ALIAS);
    FRT_CHECK(!overlaps(partials_dev, pbytes, w_packed_dev, wb), FRT_E_ALIAS);
  }
  GemmParams p{};
  p.M = M; p.N = N; p.K = K; p.MB = m_blocks(M); p.splits = splits;
  p.ab_dtype = ab_dtype; p.layout = FRT_W_PLAIN; p.ksteps_per_split = ksteps / splits;
  p.a = (const uint8_t*)a_packed_dev; p.w = (const uint8_t*)w_packed_dev; p.colscale = w_colscale_dev;
  p.act_scale = act_scale; p.act_scale_ptr = nullptr; p.partials = partials_dev; p.epi = kEpiQkv;
  p.q_out = q_out_dev; p.k_out = k_out_dev; p.v_out = v_out_dev; p.nq = n_heads * head_dim; p.hd = head_dim;
  p.v_ld = v_ld;
  hipStream_t s = (hipStream_t)stream;
  FRT_HIP(launch_gemm(p, s));
  if (splits > 1) {
    ReduceParams r{};
    r.M = M; r.N = N; r.MB = p.MB; r.splits = splits; r.partials = partials_dev;
    r.act_scale = act_scale; r.act_scale_ptr = nullptr; r.colscale = w_colscale_dev; r.epi = kEpiQkv;
    r.q_out = q_out_dev; r.k_out = k_out_dev; r.v_out = v_out_dev; r.nq = p.nq; r.hd = head_dim; r.v_ld = v_ld;
    FRT_HIP(launch_reduce(r, s));
  }
  return FRT_OK;
}
