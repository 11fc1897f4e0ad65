// Offline weight preparation and the host-side layout helpers.
//
// Pages: observation-age notes ("思考探索：具身推理加速，先看动作执行时观测有多旧"),
// section "CUDA Graph 与图化简分别省掉什么" (a fixed per-channel RMSNorm gain folds into the
// weight, W' = diag(gamma) W; rounding must be checked at low precision), section
// "静态量化改变了两次矩阵乘之间的工作" (weight scales are kept apart from the GEMM-input
// activation scales), section "小 M GEMM 要看并行度，也要看归约代价" (the skinny path keeps
// re-laid-out weight copies).
#include "frt_internal.hpp"

#include <string.h>

namespace frt {

// s_w[n] = max_k |gamma[k] * W[k][n]| / 448.  Workgroup = 64 consecutive columns (one per
// lane, so every row a wave reads is 128 contiguous bytes); its 16 waves take interleaved
// runs of 16 rows with all 16 loads in flight before the first is used, and the waves'
// maxima meet in LDS.  The products are exact in float64 (8 x 24 significand bits), a
// maximum does not depend on the order it is taken in, and the quotient is rounded once to
// fp32.  (One thread per column walking all of K left 16 waves on the whole chip for a
// 1024-column weight: 740 us per call on MI355X.)
constexpr int kColscaleWaves = 16, kColscaleRows = 16;
__global__ void __launch_bounds__(64 * kColscaleWaves) colscale_kernel(const uint16_t* __restrict__ w,
                                                                       const float* __restrict__ gamma, int K, int N,
                                                                       float* __restrict__ colscale) {
  __shared__ double part[kColscaleWaves][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = blockIdx.x * 64 + lane;
  const int nn = n < N ? n : N - 1;  // lanes past the last column read an in-bounds stand-in
  double amax = 0.0;
  for (int k0 = wave * kColscaleRows; k0 < K; k0 += kColscaleWaves * kColscaleRows) {
    double v[kColscaleRows];
#pragma unroll
    for (int e = 0; e < kColscaleRows; ++e) {
      const int k = k0 + e < K ? k0 + e : K - 1;
      v[e] = (double)bf16_to_f32(w[(size_t)k * N + nn]);
      if (gamma) v[e] *= (double)gamma[k];
    }
#pragma unroll
    for (int e = 0; e < kColscaleRows; ++e) amax = fmax(amax, fabs(v[e]));  // a repeated row changes no maximum
  }
  part[wave][lane] = amax;
  __syncthreads();
  if (wave == 0 && n < N) {
    double m = part[0][lane];
#pragma unroll
    for (int i = 1; i < kColscaleWaves; ++i) m = fmax(m, part[i][lane]);
    colscale[n] = (float)(m / 448.0);
  }
}

// One thread per 16-byte lane slot of the packed weight.
__global__ void __launch_bounds__(256) pack_weight_kernel(const uint16_t* __restrict__ w, const float* __restrict__ gamma,
                                                          int K, int N, int dtype, int layout,
                                                          const float* __restrict__ colscale, uint8_t* __restrict__ out) {
  const size_t slot = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t nslots = (size_t)K * N * (dtype == FRT_BF16 ? 2 : 1) / 16;
  if (slot >= nslots) return;
  const int KSTEP = kstep_of(dtype);
  const int KS = K / KSTEP;
  int lane, half = 0;
  size_t tile;
  if (dtype == FRT_BF16) {
    tile = slot / 64;
    lane = (int)(slot % 64);
  } else {
    tile = slot / 128;
    half = (int)((slot % 128) / 64);
    lane = (int)(slot % 64);
  }
  const int pt = (int)(tile / KS), ks = (int)(tile % KS);
  const int n = logical_tile_of(layout, N, pt) * 16 + (lane & 15);
  // first k of the slot (the operand_offset / weight_offset order)
  const int k0 = dtype == FRT_BF16 ? ks * 32 + 8 * (lane >> 4) : ks * 128 + 64 * half + 16 * (lane >> 4);
  u32x4 v;
  uint32_t* vw = reinterpret_cast<uint32_t*>(&v);
  // W' = gamma * W and W' / s_w are formed in float64 (the product is exact, the quotient
  // correctly rounded) and rounded once to the storage format
  if (dtype == FRT_BF16) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      double a = (double)bf16_to_f32(w[(size_t)(k0 + e) * N + n]);
      double b = (double)bf16_to_f32(w[(size_t)(k0 + e + 1) * N + n]);
      if (gamma) {
        a *= (double)gamma[k0 + e];
        b *= (double)gamma[k0 + e + 1];
      }
      vw[e / 2] = bf16_bits_exact(a) | (bf16_bits_exact(b) << 16);
    }
  } else {
    const double s = (double)colscale[n];
#pragma unroll
    for (int e = 0; e < 16; e += 4) {
      uint32_t word = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        double a = (double)bf16_to_f32(w[(size_t)(k0 + e + q) * N + n]);
        if (gamma) a *= (double)gamma[k0 + e + q];
        word |= (s > 0.0 ? e4m3_code_exact(a / s) : 0u) << (8 * q);
      }
      vw[e / 4] = word;
    }
  }
  *reinterpret_cast<u32x4*>(out + slot * 16) = v;
}

// FP4 E2M1 code of a float64 value: round to the nearest of the eight magnitudes
// {0, 0.5, 1, 1.5, 2, 3, 4, 6} (code order), a tie going to the even code (mantissa bit
// 0), and anything at or past 6 saturating to code 7; the sign is bit 3 (-0 keeps it).
// Counting the midpoints a magnitude passes gives the code directly.
__device__ inline uint32_t fp4_code_exact(double x) {
  const double a = fabs(x);
  const double mid[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < 7; ++i) c += (a > mid[i] || (a == mid[i] && ((i + 1) & 1) == 0)) ? 1u : 0u;
  return c | (signbit(x) ? 8u : 0u);
}

// MXFP4 weight packing: one thread per lane slot, i.e. one OCP MX block (32 consecutive
// k of one column).  W' = gamma * W is exact in float64; the block's E8M0 exponent is
// floor(log2 max|W'|) - 2 (clamped to [-127, 127]; 0 for an all-zero block) and
// W' / 2^e is exact in float64, so every code is rounded once.
__global__ void __launch_bounds__(256) pack_mxfp4_kernel(const uint16_t* __restrict__ w, const float* __restrict__ gamma,
                                                         int K, int N, int layout, uint8_t* __restrict__ out) {
  const size_t slot = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t nslots = (size_t)(K / 32) * N;
  if (slot >= nslots) return;
  const int KS = K / 128;
  const size_t tile = slot / 64;
  const int lane = (int)(slot % 64);
  const int pt = (int)(tile / KS), ks = (int)(tile % KS);
  const int n = logical_tile_of(layout, N, pt) * 16 + (lane & 15);
  const int k0 = ks * 128 + 32 * (lane >> 4);
  double v[32];
  double amax = 0.0;
#pragma unroll
  for (int q = 0; q < 32; ++q) {
    v[q] = (double)bf16_to_f32(w[(size_t)(k0 + q) * N + n]);
    if (gamma) v[q] *= (double)gamma[k0 + q];
    amax = fmax(amax, fabs(v[q]));
  }
  int e = -127;
  if (amax > 0.0) {
    int ex;
    frexp(amax, &ex);  // amax = f * 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1
    e = ex - 1 - 2;
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
  }
  u32x4 codes;
  uint32_t* cw = reinterpret_cast<uint32_t*>(&codes);
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) word |= fp4_code_exact(ldexp(v[8 * d + j], -e)) << (4 * j);
    cw[d] = word;
  }
  uint8_t* t = out + tile * 1088;
  *reinterpret_cast<u32x4*>(t + lane * 16) = codes;
  t[1024 + lane] = (uint8_t)(e + 127);
}

}  // namespace frt

using namespace frt;

extern "C" size_t frt_operand_bytes(int dtype, int M, int K) {
  if (!is_ab_dtype(dtype) || M < 1 || M > kMaxM || K < 1) return 0;
  return (size_t)m_blocks(M) * 16 * K * elem_bytes(dtype);
}

extern "C" size_t frt_weight_bytes(int dtype, int K, int N) {
  if (!is_w_dtype(dtype) || K < 1 || N < 1) return 0;
  if (dtype == FRT_MXFP4) return K % 128 ? 0 : (size_t)K * N / 2 + (size_t)(K / 32) * N;
  return (size_t)K * N * elem_bytes(dtype);
}

static int check_operand_shape(int dtype, int M, int K) {
  FRT_CHECK(is_ab_dtype(dtype), FRT_E_DTYPE);
  FRT_CHECK(M >= 1 && M <= kMaxM, FRT_E_SHAPE);
  FRT_CHECK(K >= kstep_of(dtype) && K % kstep_of(dtype) == 0, FRT_E_SHAPE);
  return FRT_OK;
}

static int check_weight_shape(int dtype, int K, int N, int layout) {
  FRT_CHECK(is_w_dtype(dtype), FRT_E_DTYPE);
  FRT_CHECK(K >= kstep_of(dtype) && K % kstep_of(dtype) == 0, FRT_E_SHAPE);
  FRT_CHECK(N >= 16 && N % 16 == 0, FRT_E_SHAPE);
  FRT_CHECK(layout == FRT_W_PLAIN || layout == FRT_W_GATE_UP, FRT_E_ARG);
  if (layout == FRT_W_GATE_UP) FRT_CHECK(N % 32 == 0, FRT_E_SHAPE);
  return FRT_OK;
}

extern "C" int frt_operand_pack_host(const void* codes_host, int dtype, int M, int K, void* packed_host) {
  FRT_CHECK(codes_host && packed_host, FRT_E_NULL);
  int st = check_operand_shape(dtype, M, K);
  if (st) return st;
  const int MB = m_blocks(M), esz = elem_bytes(dtype);
  uint8_t* out = (uint8_t*)packed_host;
  memset(out, 0, frt_operand_bytes(dtype, M, K));
  for (int m = 0; m < M; ++m)
    for (int k = 0; k < K; ++k)
      memcpy(out + operand_offset(dtype, MB, m, k), (const uint8_t*)codes_host + ((size_t)m * K + k) * esz, esz);
  return FRT_OK;
}

extern "C" int frt_operand_unpack_host(const void* packed_host, int dtype, int M, int K, void* codes_host) {
  FRT_CHECK(codes_host && packed_host, FRT_E_NULL);
  int st = check_operand_shape(dtype, M, K);
  if (st) return st;
  const int MB = m_blocks(M), esz = elem_bytes(dtype);
  for (int m = 0; m < M; ++m)
    for (int k = 0; k < K; ++k)
      memcpy((uint8_t*)codes_host + ((size_t)m * K + k) * esz, (const uint8_t*)packed_host + operand_offset(dtype, MB, m, k), esz);
  return FRT_OK;
}

extern "C" int frt_weight_pack_host(const void* codes_host, int dtype, int K, int N, int layout, void* packed_host) {
  FRT_CHECK(codes_host && packed_host, FRT_E_NULL);
  FRT_CHECK(is_ab_dtype(dtype), FRT_E_DTYPE);  // MXFP4: frt_weight_pack_mxfp4_host
  int st = check_weight_shape(dtype, K, N, layout);
  if (st) return st;
  const int esz = elem_bytes(dtype);
  for (int k = 0; k < K; ++k)
    for (int n = 0; n < N; ++n)
      memcpy((uint8_t*)packed_host + weight_offset(dtype, layout, K, N, k, n),
             (const uint8_t*)codes_host + ((size_t)k * N + n) * esz, esz);
  return FRT_OK;
}

extern "C" int frt_weight_unpack_host(const void* packed_host, int dtype, int K, int N, int layout, void* codes_host) {
  FRT_CHECK(codes_host && packed_host, FRT_E_NULL);
  FRT_CHECK(is_ab_dtype(dtype), FRT_E_DTYPE);
  int st = check_weight_shape(dtype, K, N, layout);
  if (st) return st;
  const int esz = elem_bytes(dtype);
  for (int k = 0; k < K; ++k)
    for (int n = 0; n < N; ++n)
      memcpy((uint8_t*)codes_host + ((size_t)k * N + n) * esz,
             (const uint8_t*)packed_host + weight_offset(dtype, layout, K, N, k, n), esz);
  return FRT_OK;
}

extern "C" int frt_weight_pack_mxfp4_host(const uint8_t* codes_host, const uint8_t* scales_host, int K, int N,
                                          int layout, void* packed_host) {
  FRT_CHECK(codes_host && scales_host && packed_host, FRT_E_NULL);
  int st = check_weight_shape(FRT_MXFP4, K, N, layout);
  if (st) return st;
  uint8_t* out = (uint8_t*)packed_host;
  memset(out, 0, frt_weight_bytes(FRT_MXFP4, K, N));
  for (int k = 0; k < K; ++k)
    for (int n = 0; n < N; ++n) {
      const uint32_t c = codes_host[(size_t)k * N + n] & 15u;
      out[mx_code_byte(layout, K, N, k, n)] |= (uint8_t)(c << (4 * (k & 1)));
      if (k % 32 == 0) out[mx_scale_byte(layout, K, N, k, n)] = scales_host[(size_t)(k / 32) * N + n];
    }
  return FRT_OK;
}

extern "C" int frt_weight_unpack_mxfp4_host(const void* packed_host, int K, int N, int layout, uint8_t* codes_host,
                                            uint8_t* scales_host) {
  FRT_CHECK(codes_host && scales_host && packed_host, FRT_E_NULL);
  int st = check_weight_shape(FRT_MXFP4, K, N, layout);
  if (st) return st;
  const uint8_t* in = (const uint8_t*)packed_host;
  for (int k = 0; k < K; ++k)
    for (int n = 0; n < N; ++n) {
      codes_host[(size_t)k * N + n] = (uint8_t)((in[mx_code_byte(layout, K, N, k, n)] >> (4 * (k & 1))) & 15u);
      if (k % 32 == 0) scales_host[(size_t)(k / 32) * N + n] = in[mx_scale_byte(layout, K, N, k, n)];
    }
  return FRT_OK;
}

extern "C" int frt_pack_weight(void* stream, int K, int N, const uint16_t* w_bf16_dev, const float* gamma_dev,
                               int dtype, int layout, void* w_packed_dev, float* colscale_dev) {
  FRT_CHECK(w_bf16_dev && w_packed_dev, FRT_E_NULL);
  int st = check_weight_shape(dtype, K, N, layout);
  if (st) return st;
  if (dtype == FRT_E4M3) FRT_CHECK(colscale_dev, FRT_E_NULL);
  const void* ptrs[] = {w_bf16_dev, gamma_dev, w_packed_dev, dtype == FRT_E4M3 ? colscale_dev : nullptr};
  for (const void* q : ptrs) FRT_CHECK(aligned16(q), FRT_E_ALIGN);
  const size_t wb = (size_t)K * N * 2, pb = frt_weight_bytes(dtype, K, N);
  FRT_CHECK(!overlaps(w_bf16_dev, wb, w_packed_dev, pb), FRT_E_ALIAS);
  if (dtype == FRT_E4M3) {
    FRT_CHECK(!overlaps(colscale_dev, (size_t)N * 4, w_packed_dev, pb), FRT_E_ALIAS);
    FRT_CHECK(!overlaps(colscale_dev, (size_t)N * 4, w_bf16_dev, wb), FRT_E_ALIAS);
  }
  hipStream_t s = (hipStream_t)stream;
  if (dtype == FRT_MXFP4) {
    const size_t nslots = (size_t)(K / 32) * N;
    hipLaunchKernelGGL(pack_mxfp4_kernel, dim3((unsigned)((nslots + 255) / 256)), dim3(256), 0, s, w_bf16_dev,
                       gamma_dev, K, N, layout, (uint8_t*)w_packed_dev);
    FRT_HIP(hipGetLastError());
    return FRT_OK;
  }
  if (dtype == FRT_E4M3) {
    hipLaunchKernelGGL(colscale_kernel, dim3((N + 63) / 64), dim3(64 * kColscaleWaves), 0, s, w_bf16_dev, gamma_dev,
                       K, N, colscale_dev);
    FRT_HIP(hipGetLastError());
  }
  const size_t nslots = pb / 16;
  hipLaunchKernelGGL(pack_weight_kernel, dim3((unsigned)((nslots + 255) / 256)), dim3(256), 0, s, w_bf16_dev, gamma_dev,
                     K, N, dtype, layout, (const float*)colscale_dev, (uint8_t*)w_packed_dev);
  FRT_HIP(hipGetLastError());
  return FRT_OK;
}
