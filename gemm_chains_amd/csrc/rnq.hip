// Producer: [split-K reduce + scale recovery] -> gated residual -> (Ada)RMSNorm ->
// static-scale quantisation, written straight into the packed operand of the next GEMM.
//
// Pages: observation-age notes ("思考探索：具身推理加速，先看动作执行时观测有多旧"),
// section "CUDA Graph 与图化简分别省掉什么" (RMSNorm: xhat = x / sqrt(mean(x^2) + eps)),
// section "静态量化改变了两次矩阵乘之间的工作" (scale fixed ahead of the run; gated residual,
// AdaRMSNorm and FP8 conversion fused; the consumer of layer l prepares layer l+1's input
// with layer l+1's conditioning), section "小 M GEMM 要看并行度，也要看归约代价" (the next
// consumer reduces the FP32 partial sums); rebasdaily FlashRT-PAI news summary, section
// "它优化的是“接力方式”" (the producer's output layout is exactly what the GEMM reads).
//
// One 256-thread workgroup owns one row (Mp workgroups), so a row's loads are spread over
// four waves and issued together: each thread keeps groups of 4 consecutive k in
// registers (one group per 1024 of K), the sum of squares is reduced with a fixed
// butterfly inside each wave and then across the four waves in wave order (bitwise
// deterministic), and each group is written as one 8-byte (bf16) or 4-byte (e4m3) piece of
// a lane slot of the packed operand.  Rows M..Mp-1 write zero codes so the GEMM can always
// read whole 16-row blocks.
#include "frt_internal.hpp"

namespace frt {

// Kernel variants are compile-time in everything that shapes the code: SPL = number of
// fp32 partial slices read (0: no x; -1: any count, run-time loop), G = groups of 4
// elements per thread (K <= 1024 G), ODT = output operand format (0: none).  Every
// launch fetches its code cold, so each variant carries only its own path.  All of a
// group's loads are issued before the first is used: the partials come from the previous
// kernel and sit beyond this XCD's L2.
template <int SPL, int G, int ODT>
__global__ void __launch_bounds__(256) rnq_kernel(const RnqParams p) {
  const int m = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int K = p.K;
  __shared__ float wsum[4];
  const int rows = p.operand ? p.MB * 16 : p.M;
  if (__builtin_expect(m >= rows, 0)) {  // extra workgroups: read the following GEMMs' weights ahead
    const unsigned v = touch_weights(p.touch, m, rows, p.touch_wgs);
    if (v == 0x9e3779b9u && p.sink) *p.sink = v;  // practically never taken
    return;
  }
  if (__builtin_expect(m >= p.M, 0)) {  // padding rows of the operand: zero codes (only with an operand)
    if constexpr (ODT != 0) {
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const int k0 = 4 * (tid + 256 * i);
        if (k0 < K) store_operand4(p.operand, ODT, p.MB, m, k0, 0.f, 0.f, 0.f, 0.f, 1.f, true);
      }
    }
    return;
  }
  const size_t row = (size_t)m * K;
  const size_t split_stride = (size_t)p.M * K;

  // Every input of the row is requested before the first one is used: the partials, the
  // residual, the per-channel vectors and the scalar scales.  (Loads behind a null test
  // would each wait for the data before them, and loads after the barrier below would
  // cost one more memory round trip each.)  A missing vector reads the residual's row
  // in its place, which is always valid, and its value is then not used.
  const bool has_cs = p.x_colscale != nullptr, has_gate = p.gate != nullptr;
  const bool has_as = p.ada_scale != nullptr, has_sh = p.ada_shift != nullptr;
  const float* csp = has_cs ? p.x_colscale : p.residual;
  const float* gtp = has_gate ? p.gate : p.residual;
  const float* asp = has_as ? p.ada_scale : p.residual;
  const float* shp = has_sh ? p.ada_shift : p.residual;
  const float xs = SPL != 0 ? load_scale(p.x_scale_ptr, p.x_scale) : 1.f;
  const float as = load_scale(p.act_scale_ptr, p.act_scale);
  f32x4 r[G], xp[G][SPL > 0 ? SPL : 1], cs[G], gt[G], av[G], sv[G];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const int k0 = 4 * (tid + 256 * i);
    if (k0 >= K) continue;
    r[i] = *reinterpret_cast<const f32x4*>(p.residual + row + k0);
    if constexpr (SPL > 0) {
#pragma unroll
      for (int j = 0; j < SPL; ++j) xp[i][j] = *reinterpret_cast<const f32x4*>(p.x + j * split_stride + row + k0);
    }
    if constexpr (SPL != 0) {
      cs[i] = *reinterpret_cast<const f32x4*>(csp + k0);
      gt[i] = *reinterpret_cast<const f32x4*>(gtp + k0);
    }
    if constexpr (ODT != 0) {
      av[i] = *reinterpret_cast<const f32x4*>(asp + k0);
      sv[i] = *reinterpret_cast<const f32x4*>(shp + k0);
    }
  }

  f32x4 h[G];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const int k0 = 4 * (tid + 256 * i);
    if (k0 >= K) {
      h[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      continue;
    }
    f32x4 hv = r[i];
    if constexpr (SPL != 0) {
      f32x4 x;
      if constexpr (SPL > 0) {
        x = xp[i][0];
#pragma unroll
        for (int j = 1; j < SPL; ++j) x += xp[i][j];  // partials summed in ascending split order
      } else {
        x = *reinterpret_cast<const f32x4*>(p.x + row + k0);
        for (int j = 1; j < p.x_splits; ++j) x += *reinterpret_cast<const f32x4*>(p.x + j * split_stride + row + k0);
      }
      x *= xs;  // then scale recovery
      if (has_cs) x *= cs[i];
      if (has_gate) x *= gt[i];
      hv = hv + x;
    }
    h[i] = hv;
#pragma unroll
    for (int e = 0; e < 4; ++e) ss = fmaf(hv[e], hv[e], ss);
  }
  if (p.residual_out) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int k0 = 4 * (tid + 256 * i);
      if (k0 < K) *reinterpret_cast<f32x4*>(p.residual_out + row + k0) = h[i];
    }
  }
  if constexpr (ODT != 0) {
    // xor butterfly 32, 16, 8, 4, 2, 1 on the VALU (bitwise the __shfl_xor butterfly)
    ss = xor_add<32>(ss);
    ss = xor_add<16>(ss);
    ss = xor_add<8>(ss);
    ss = xor_add<4>(ss);
    ss = xor_add<2>(ss);
    ss = xor_add<1>(ss);
    if (lane == 0) wsum[wave] = ss;
    __syncthreads();
    const float tot = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
    const float inv = 1.0f / sqrtf(tot / (float)K + p.eps);
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int k0 = 4 * (tid + 256 * i);
      if (k0 >= K) continue;
      f32x4 y = h[i] * inv;
      if (has_as) y = y * (1.0f + av[i]);
      if (has_sh) y = y + sv[i];
      store_operand4(p.operand, ODT, p.MB, m, k0, y.x, y.y, y.z, y.w, as, false);
      record_amax(p.amax, y.x, y.y, y.z, y.w);
    }
  }
}

template <int SPL, int G>
static void launch_odt(const RnqParams& p, dim3 g, dim3 b, hipStream_t s) {
  if (!p.operand) hipLaunchKernelGGL((rnq_kernel<SPL, G, 0>), g, b, 0, s, p);
  else if (p.out_dtype == FRT_BF16) hipLaunchKernelGGL((rnq_kernel<SPL, G, FRT_BF16>), g, b, 0, s, p);
  else hipLaunchKernelGGL((rnq_kernel<SPL, G, FRT_E4M3>), g, b, 0, s, p);
}

template <int SPL>
static void launch_g(const RnqParams& p, dim3 g, dim3 b, hipStream_t s) {
  switch ((p.K + 1023) / 1024) {
    case 1: launch_odt<SPL, 1>(p, g, b, s); break;
    case 2: launch_odt<SPL, 2>(p, g, b, s); break;
    case 3: launch_odt<SPL, 3>(p, g, b, s); break;
    default: launch_odt<SPL, 4>(p, g, b, s); break;
  }
}

hipError_t launch_rnq(const RnqParams& p, hipStream_t s) {
  const int rows = p.operand ? p.MB * 16 : p.M;
  const dim3 g(rows + p.touch_wgs), b(256);
  switch (p.x ? p.x_splits : 0) {
    case 0: launch_g<0>(p, g, b, s); break;
    case 1: launch_g<1>(p, g, b, s); break;
    case 2: launch_g<2>(p, g, b, s); break;
    case 4: launch_g<4>(p, g, b, s); break;
    case 8: launch_g<8>(p, g, b, s); break;
    case 16: launch_g<16>(p, g, b, s); break;
    default: launch_g<-1>(p, g, b, s); break;
  }
  return hipGetLastError();
}

}  // namespace frt

using namespace frt;

extern "C" int frt_residual_norm_quant(void* stream, int M, int K, const float* x_dev, int x_splits,
                                       float x_scale, const float* x_colscale_dev,
                                       const float* residual_dev, float* residual_out_dev,
                                       const float* gate_dev, const float* ada_scale_dev,
                                       const float* ada_shift_dev, float eps, int out_dtype,
                                       float act_scale, void* operand_out_dev) {
  FRT_CHECK(residual_dev, FRT_E_NULL);
  FRT_CHECK(operand_out_dev || residual_out_dev, FRT_E_NULL);
  FRT_CHECK(M >= 1 && M <= kMaxM, FRT_E_SHAPE);
  FRT_CHECK(K >= 16 && K <= kMaxProducerK && K % 16 == 0, FRT_E_SHAPE);
  if (operand_out_dev) {
    FRT_CHECK(is_ab_dtype(out_dtype), FRT_E_DTYPE);
    FRT_CHECK(K % kstep_of(out_dtype) == 0, FRT_E_SHAPE);
    if (out_dtype == FRT_E4M3) FRT_CHECK(act_scale > 0.f && act_scale < __builtin_huge_valf(), FRT_E_ARG);
  }
  if (x_dev) FRT_CHECK(x_splits >= 1 && x_splits <= kMaxSplits, FRT_E_SPLITK);
  FRT_CHECK(eps >= 0.f && eps == eps, FRT_E_ARG);
  const void* ptrs[] = {x_dev, x_colscale_dev, residual_dev, residual_out_dev, gate_dev,
                        ada_scale_dev, ada_shift_dev, operand_out_dev};
  for (const void* q : ptrs) FRT_CHECK(aligned16(q), FRT_E_ALIGN);
  const size_t mk = (size_t)M * K * 4;
  const size_t opb = operand_out_dev ? frt_operand_bytes(out_dtype, M, K) : 0;
  // the residual may be updated in place; every other output must stand apart
  FRT_CHECK(!overlaps(operand_out_dev, opb, residual_dev, mk), FRT_E_ALIAS);
  FRT_CHECK(!overlaps(operand_out_dev, opb, residual_out_dev, mk), FRT_E_ALIAS);
  if (x_dev) {
    const size_t xb = mk * (size_t)x_splits;
    FRT_CHECK(!overlaps(operand_out_dev, opb, x_dev, xb), FRT_E_ALIAS);
    FRT_CHECK(!overlaps(residual_out_dev, mk, x_dev, xb), FRT_E_ALIAS);
  }
  if (residual_out_dev && residual_out_dev != residual_dev)
    FRT_CHECK(!overlaps(residual_out_dev, mk, residual_dev, mk), FRT_E_ALIAS);

  RnqParams p{};
  p.M = M; p.K = K; p.MB = m_blocks(M);
  p.x = x_dev; p.x_splits = x_dev ? x_splits : 0; p.x_scale = x_scale; p.x_scale_ptr = nullptr;
  p.x_colscale = x_colscale_dev; p.residual = residual_dev; p.residual_out = residual_out_dev;
  p.gate = gate_dev; p.ada_scale = ada_scale_dev; p.ada_shift = ada_shift_dev; p.eps = eps;
  p.out_dtype = operand_out_dev ? out_dtype : FRT_BF16;
  p.act_scale = out_dtype == FRT_E4M3 ? act_scale : 1.0f; p.act_scale_ptr = nullptr;
  p.operand = (uint8_t*)operand_out_dev;
  FRT_HIP(launch_rnq(p, (hipStream_t)stream));
  return FRT_OK;
}
