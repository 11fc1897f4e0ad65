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
#include "gemm_kernel.hpp"

#include <mutex>

namespace frt {

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
// Frag registers per lane and k-step: 4 (bf16), 8 (e4m3), 5 (MXFP4 codes + scale) per
// weight tile, 4 or 8 per operand tile.  A round's loads stay within ~192 VGPRs so that
// every one of them can be in flight at once.
static int per_max(int dtype, int nt, int mbw) {
  const int v = nt * frag_regs(dtype) + mbw * frag_regs(act_dtype_of(dtype));
  int per = 8;
  while (per > 1 && per * v > 192) per /= 2;
  return per;
}

// Measured on MI355X at the action-decoder shapes (M = 10/50, K = 1024..4096) and the
// K = 2048, N = 16384 gate|up sweep:
//  - widest column group (NT = 4, 2, 1) that still leaves >= 512 workgroups, i.e. two
//    per CU: a read-rate probe of the GEMM's own weight pattern streams 64 MB at 5.7 TB/s
//    with 512 workgroups of 2 tiles against 4.6 TB/s with 256 of 4 (the same bytes in
//    flight per CU, twice the waves); the sweep's bf16 GEMM at M <= 16 went from 15.9 to
//    12.8 us, e4m3 from 8.1-11.0 to 7.7-10.0 us, and every chain by 0.1-0.5 us/layer (the
//    down projection).  MXFP4 weights with the SiLU epilogue keep >= 256 (5.25 against
//    5.5 us at M = 1): their 1088-byte tiles are small next to the activation tiles every
//    extra workgroup re-reads.  The SiLU epilogue needs gate/up pairs (even NT);
//  - when even the narrowest group leaves fewer than 256 workgroups, the row blocks are
//    spread over row groups (one block each) on the column group's XCD;
//  - four waves per workgroup, each with as many k-steps per round as its registers
//    allow (eight waves with shorter runs lose to the longer LDS merge).
static GemmShape choose_shape(const GemmParams& p) {
  GemmShape sh{};
  const int tiles = p.N / 16;
  const bool partial = p.epi == FRT_EPI_NONE || p.splits > 1;
  if (partial) sh.epi = kGemmPartial;
  else if (p.epi == FRT_EPI_SILU_GATE_QUANT) sh.epi = p.out_dtype == FRT_BF16 ? kGemmSiluBf16 : kGemmSiluE4m3;
  else sh.epi = p.epi == kEpiQkv ? kGemmQkv : kGemmStore;
  const int nt_min = sh.epi == kGemmSiluBf16 || sh.epi == kGemmSiluE4m3 ? 2 : 1;
  sh.nt = nt_min;
  const int wg_target = p.ab_dtype == FRT_MXFP4 && nt_min == 2 ? 256 : 512;
  for (int cand : {4, 2}) {
    if (tiles % cand || cand < nt_min) continue;
    if ((tiles / cand) * p.splits >= wg_target) { sh.nt = cand; break; }
  }
  if (tiles % sh.nt) sh.nt = 1;
  sh.col_groups = tiles / sh.nt;
  sh.mbw = p.MB;
  sh.row_groups = 1;
  if (sh.col_groups * p.splits < 256 && p.MB > 1) {
    sh.mbw = 1;
    sh.row_groups = p.MB;
  }
  const int kps = p.ksteps_per_split;
  sh.kw = kps % 4 == 0 ? 4 : (kps % 2 == 0 ? 2 : 1);
  const int run = kps / sh.kw;
  sh.per = per_max(p.ab_dtype, sh.nt, sh.mbw);
  while (sh.per > 1 && run % sh.per) sh.per /= 2;
  const bool scaled = sh.epi != kGemmPartial &&
                      (p.act_scale_ptr || p.colscale || p.out_scale_ptr || p.amax);
  sh.fast = sh.kw == 4 && run == sh.per ? (scaled ? kFastShape : kFastPlain) : kGeneric;
  return sh;
}

WeightTouch gemm_weight_touch(const GemmParams& p, int part, int parts) {
  const GemmShape sh = choose_shape(p);
  WeightTouch t{};
  t.w = p.w;
  t.tb = tile_bytes_of(p.ab_dtype);
  t.ks = p.K / kstep_of(p.ab_dtype);
  t.nt = sh.nt;
  t.kps = p.ksteps_per_split;
  t.col_groups = sh.col_groups;
  t.row_groups = sh.row_groups;
  t.splits = p.splits;
  t.part = part;
  t.parts = parts;
  return t;
}

// The kernels are compiled in the gemm_{bf16,e4m3,mxfp4}{,_silu}.hip units, not here.
#define FRT_GEMM_EXTERN(DT)                                                                              \
  extern template hipError_t launch_gemm_epi<DT, kGemmPartial>(const GemmParams&, const GemmShape&, hipStream_t); \
  extern template hipError_t launch_gemm_epi<DT, kGemmStore>(const GemmParams&, const GemmShape&, hipStream_t);   \
  extern template hipError_t launch_gemm_epi<DT, kGemmQkv>(const GemmParams&, const GemmShape&, hipStream_t);     \
  extern template hipError_t launch_gemm_epi<DT, kGemmSiluBf16>(const GemmParams&, const GemmShape&, hipStream_t); \
  extern template hipError_t launch_gemm_epi<DT, kGemmSiluE4m3>(const GemmParams&, const GemmShape&, hipStream_t);
FRT_GEMM_EXTERN(FRT_BF16)
FRT_GEMM_EXTERN(FRT_E4M3)
FRT_GEMM_EXTERN(FRT_MXFP4)
#undef FRT_GEMM_EXTERN

template <int DT>
static hipError_t launch_gemm_dt(const GemmParams& p, const GemmShape& sh, hipStream_t s) {
  switch (sh.epi) {
    case kGemmPartial: return launch_gemm_epi<DT, kGemmPartial>(p, sh, s);
    case kGemmStore: return launch_gemm_epi<DT, kGemmStore>(p, sh, s);
    case kGemmSiluBf16: return launch_gemm_epi<DT, kGemmSiluBf16>(p, sh, s);
    case kGemmSiluE4m3: return launch_gemm_epi<DT, kGemmSiluE4m3>(p, sh, s);
    default: return launch_gemm_epi<DT, kGemmQkv>(p, sh, s);
  }
}

hipError_t launch_gemm(const GemmParams& p_in, hipStream_t s) {
  GemmParams p = p_in;
  const GemmShape sh = choose_shape(p);
  p.kwaves = sh.kw;
  p.run = p.ksteps_per_split / sh.kw;
  p.ksteps = p.K / kstep_of(p.ab_dtype);
  p.row_groups = sh.row_groups;
  p.col_groups = sh.col_groups;
  switch (p.ab_dtype) {
    case FRT_BF16: return launch_gemm_dt<FRT_BF16>(p, sh, s);
    case FRT_E4M3: return launch_gemm_dt<FRT_E4M3>(p, sh, s);
    default: return launch_gemm_dt<FRT_MXFP4>(p, sh, s);
  }
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
// partials are the output (the next producer reduces them anyway), split until one
// column tile per workgroup gives 256 workgroups, keeping >= 4 k-steps per chunk.  Every
// split adds an M x N fp32 slice that the consumer reads back; in the chain's down
// projection (K = 4096, N = 1024, M = 50/10, bf16 and e4m3) 4 splits beat 8 by
// 0.2-0.7 us per layer and 16 lost 1.2-2.6 us.
int choose_splits(int M, int N, int K, int dtype, int epi) {
  (void)M;
  if (epi != FRT_EPI_NONE) return 1;
  const int tiles = N / 16;
  const int ksteps = K / kstep_of(dtype);
  int s = 1;
  while (s < 16 && tiles * s < 256 && ksteps % (2 * s) == 0 && ksteps / (2 * s) >= 4) s *= 2;
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
  if (M < 1 || M > kMaxM || N < 16 || N % 16 || !is_w_dtype(ab_dtype) || K < kstep_of(ab_dtype) ||
      K % kstep_of(ab_dtype))
    return 0;
  return choose_splits(M, N, K, ab_dtype, FRT_EPI_NONE);
}

// Argument checks of the skinny GEMM entry points (no HIP call).  `splits` is resolved in
// place (0 = the library's choice).  With scratch_partials the partial sums go to the
// library's own scratch array, so the caller's partials arguments are not checked.
static int gemm_validate(int M, int N, int K, int& splits, int ab_dtype, int layout, const void* a_packed_dev,
                         const void* w_packed_dev, const float* w_colscale_dev, float act_scale,
                         const float* partials_dev, size_t partials_bytes, bool scratch_partials, int epi,
                         const void* out_dev, int out_dtype, float out_act_scale) {
  FRT_CHECK(a_packed_dev && w_packed_dev, FRT_E_NULL);
  FRT_CHECK(is_w_dtype(ab_dtype), FRT_E_DTYPE);
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
  if (epi == FRT_EPI_SILU_GATE_QUANT) FRT_CHECK(layout == FRT_W_GATE_UP || splits > 1, FRT_E_ARG);
  int st = validate_epilogue_out(M, N, epi, out_dev, out_dtype, out_act_scale);
  if (st != FRT_OK) return st;
  const void* ptrs[] = {a_packed_dev, w_packed_dev, w_colscale_dev, scratch_partials ? nullptr : partials_dev};
  for (const void* q : ptrs) FRT_CHECK(aligned16(q), FRT_E_ALIGN);
  const bool need_partials = epi == FRT_EPI_NONE || splits > 1;
  const size_t pbytes = (size_t)splits * M * N * 4;
  if (need_partials && !scratch_partials) {
    FRT_CHECK(partials_dev, FRT_E_NULL);
    FRT_CHECK(partials_bytes >= pbytes, FRT_E_WORKSPACE);
  }
  const size_t ab = frt_operand_bytes(act_dtype_of(ab_dtype), M, K);
  const size_t wb = frt_weight_bytes(ab_dtype, K, N);
  const size_t ob = epilogue_out_bytes(M, N, epi, out_dtype);
  if (need_partials && !scratch_partials) {
    FRT_CHECK(!overlaps(partials_dev, pbytes, a_packed_dev, ab), FRT_E_ALIAS);
    FRT_CHECK(!overlaps(partials_dev, pbytes, w_packed_dev, wb), FRT_E_ALIAS);
    FRT_CHECK(!overlaps(partials_dev, pbytes, out_dev, ob), FRT_E_ALIAS);
  }
  FRT_CHECK(!overlaps(out_dev, ob, a_packed_dev, ab), FRT_E_ALIAS);
  FRT_CHECK(!overlaps(out_dev, ob, w_packed_dev, wb), FRT_E_ALIAS);
  return FRT_OK;
}

// The GEMM (and, when split with an epilogue, its consumer) on validated arguments.
static int gemm_enqueue(hipStream_t s, int M, int N, int K, int splits, int ab_dtype, int layout,
                        const void* a_packed_dev, const void* w_packed_dev, const float* w_colscale_dev,
                        float act_scale, float* partials_dev, int epi, void* out_dev, int out_dtype,
                        float out_act_scale) {
  GemmParams p{};
  p.M = M; p.N = N; p.K = K; p.MB = m_blocks(M); p.splits = splits;
  p.ab_dtype = ab_dtype; p.layout = layout; p.ksteps_per_split = K / kstep_of(ab_dtype) / splits;
  p.a = (const uint8_t*)a_packed_dev; p.w = (const uint8_t*)w_packed_dev; p.colscale = w_colscale_dev;
  p.act_scale = act_scale; p.act_scale_ptr = nullptr; p.partials = partials_dev;
  p.epi = epi; p.out = out_dev; p.out_dtype = out_dtype; p.out_scale = out_dtype == FRT_E4M3 ? out_act_scale : 1.f;
  p.out_scale_ptr = nullptr;
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

extern "C" int frt_skinny_gemm_splitk(void* stream, int M, int N, int K, int splits, int ab_dtype,
                                      int layout, const void* a_packed_dev, const void* w_packed_dev,
                                      const float* w_colscale_dev, float act_scale, float* partials_dev,
                                      size_t partials_bytes, int epi, void* out_dev, int out_dtype,
                                      float out_act_scale) {
  const int st = gemm_validate(M, N, K, splits, ab_dtype, layout, a_packed_dev, w_packed_dev, w_colscale_dev,
                               act_scale, partials_dev, partials_bytes, false, epi, out_dev, out_dtype,
                               out_act_scale);
  if (st != FRT_OK) return st;
  return gemm_enqueue((hipStream_t)stream, M, N, K, splits, ab_dtype, layout, a_packed_dev, w_packed_dev,
                      w_colscale_dev, act_scale, partials_dev, epi, out_dev, out_dtype, out_act_scale);
}

// ------------------------------------------------------------------ allocation-free variant
// For callers that cannot allocate device memory (code under graph capture, tight serving
// loops): the split-K partials of frt_skinny_gemm_splitk_noalloc live in this file-scope
// array, one copy per GPU, held from the library's load until the process ends.  Host
// code never uses the array's name as an address: the device address of each GPU's copy
// comes from hipGetSymbolAddress, once per device (on the first call made with that
// device current), and is kept per device.  Every call on a GPU shares its copy, so calls
// that overlap in time on one GPU race; the partials are fully rewritten by every call
// that uses them (nothing needs clearing).
constexpr size_t kScratchBytes = (size_t)16 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

static std::mutex g_scratch_mu;
static void* g_scratch_dev[kMaxDevices] = {};

static int scratch_of_current_device(float** out) {
  int dev = -1;
  FRT_HIP(hipGetDevice(&dev));
  FRT_CHECK(dev >= 0 && dev < kMaxDevices, FRT_E_STATE);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    FRT_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    FRT_CHECK(p != nullptr, FRT_E_HIP);
    g_scratch_dev[dev] = p;
  }
  *out = static_cast<float*>(g_scratch_dev[dev]);
  return FRT_OK;
}

extern "C" size_t frt_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" int frt_skinny_gemm_splitk_noalloc(void* stream, int M, int N, int K, int splits, int ab_dtype,
                                              int layout, const void* a_packed_dev, const void* w_packed_dev,
                                              const float* w_colscale_dev, float act_scale, int epi,
                                              void* out_dev, int out_dtype, float out_act_scale) {
  FRT_CHECK(epi == FRT_EPI_STORE_F32 || epi == FRT_EPI_STORE_BF16 || epi == FRT_EPI_SILU_GATE_QUANT, FRT_E_ARG);
  int st = gemm_validate(M, N, K, splits, ab_dtype, layout, a_packed_dev, w_packed_dev, w_colscale_dev, act_scale,
                         nullptr, 0, true, epi, out_dev, out_dtype, out_act_scale);
  if (st != FRT_OK) return st;
  FRT_CHECK((size_t)splits * M * N * 4 <= kScratchBytes, FRT_E_WORKSPACE);
  float* partials = nullptr;
  if (splits > 1) {
    st = scratch_of_current_device(&partials);
    if (st != FRT_OK) return st;
  }
  return gemm_enqueue((hipStream_t)stream, M, N, K, splits, ab_dtype, layout, a_packed_dev, w_packed_dev,
                      w_colscale_dev, act_scale, partials, epi, out_dev, out_dtype, out_act_scale);
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
  FRT_CHECK(is_w_dtype(ab_dtype), FRT_E_DTYPE);
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
  const size_t ab = frt_operand_bytes(act_dtype_of(ab_dtype), M, K), wb = frt_weight_bytes(ab_dtype, K, N);
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
