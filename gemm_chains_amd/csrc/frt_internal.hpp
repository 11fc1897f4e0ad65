// Internal helpers shared by the kernels and the C ABI of the action-decoder chain.
// gfx950 (CDNA4) only: wave64, MFMA 16x16x32 bf16 and 16x16x128 f8f6f4.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/frt.h"

namespace frt {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

constexpr int kMaxM = 64;
constexpr int kMaxSplits = 16;
constexpr int kMaxProducerK = 4096;

// ------------------------------------------------------------------ status plumbing
void set_hip_error(int e);
#define FRT_HIP(call)                                  \
  do {                                                 \
    hipError_t e_ = (call);                            \
    if (e_ != hipSuccess) {                            \
      frt::set_hip_error((int)e_);                     \
      return FRT_E_HIP;                                \
    }                                                  \
  } while (0)
#define FRT_CHECK(cond, code) \
  do {                        \
    if (!(cond)) return (code); \
  } while (0)

inline bool aligned16(const void* p) { return (((uintptr_t)p) & 15u) == 0; }
inline int elem_bytes(int dtype) { return dtype == FRT_BF16 ? 2 : (dtype == FRT_E4M3 ? 1 : 4); }
inline bool is_ab_dtype(int dtype) { return dtype == FRT_BF16 || dtype == FRT_E4M3; }
// Weight formats of a GEMM, and the operand (activation) format each one multiplies.
inline bool is_w_dtype(int dtype) { return is_ab_dtype(dtype) || dtype == FRT_MXFP4; }
__host__ __device__ constexpr int act_dtype_of(int wdtype) { return wdtype == FRT_MXFP4 ? FRT_E4M3 : wdtype; }
inline bool is_split(int s) { return s == 1 || s == 2 || s == 4 || s == 8 || s == 16; }
inline int m_blocks(int M) { return (M + 15) / 16; }
// Elements of K covered by one MFMA k-step (and one packed tile): 32 bf16, 128 e4m3/MXFP4.
__host__ __device__ constexpr int kstep_of(int dtype) { return dtype == FRT_BF16 ? 32 : 128; }
// Bytes of one packed tile (16 rows or columns x one k-step).
__host__ __device__ constexpr int tile_bytes_of(int dtype) {
  return dtype == FRT_BF16 ? 1024 : (dtype == FRT_MXFP4 ? 1088 : 2048);
}
inline bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// ------------------------------------------------------------------ packed layouts
// Packed GEMM operand (activations), Mp = 16*MB rows, logical A[m][k]:
//   one tile per (m-block mb, k-step ks) at byte (ks*MB + mb)*TB, so the MB tiles a GEMM
//   wave needs for one k-step are adjacent.  Inside a tile, MFMA lane L (0..63) owns row
//   m = 16*mb + L%16 and, with g = L/16:
//   - bf16 (k-step 32): the 16 bytes at L*16, k = ks*32 + 8g + [0, 8);
//   - e4m3 (k-step 128): two 16-byte halves h at h*1024 + L*16, half h holding
//     k = ks*128 + 64h + 16g + [0, 16).  (This order makes the 32 FP4 elements an MXFP4
//     weight lane pairs with, measured on gfx950's FP4 x FP8 block-scaled MFMA, the
//     contiguous k range 32g' + [0, 32) of weight lane group g' -- one OCP MX block, under
//     that lane's scale.  FP8 x FP8 pairs byte p of A lane L with byte p of B lane L, so
//     any order shared by both operands gives the same contraction.)
__host__ __device__ inline size_t operand_offset(int dtype, int MB, int m, int k) {
  const int mb = m >> 4, r = m & 15;
  if (dtype == FRT_BF16) {
    const int ks = k >> 5, kk = k & 31;
    const int lane = r + 16 * (kk >> 3);
    return ((size_t)ks * MB + mb) * 1024 + (size_t)lane * 16 + (size_t)(kk & 7) * 2;
  }
  const int ks = k >> 7, kk = k & 127;
  const int lane = r + 16 * ((kk >> 4) & 3);
  const int half = kk >> 6;
  return ((size_t)ks * MB + mb) * 2048 + (size_t)half * 1024 + (size_t)lane * 16 + (kk & 15);
}

// Packed weight, logical W[k][n]: the MFMA's A operand is a W^T tile of 16 output
// columns x one k-step.  Tile (packed column tile pt, k-step ks) sits at byte
// (pt*KSTEPS + ks)*TB (column-tile major, so a workgroup's share is contiguous); lane L
// holds column n = 16*lt + L%16 of logical tile lt and the same k positions as above.
__host__ __device__ inline int packed_tile_of(int layout, int N, int lt) {
  if (layout == FRT_W_GATE_UP) {
    const int half_tiles = N / 32;
    return lt < half_tiles ? 2 * lt : 2 * (lt - half_tiles) + 1;
  }
  return lt;
}
__host__ __device__ inline int logical_tile_of(int layout, int N, int pt) {
  if (layout == FRT_W_GATE_UP) return (pt & 1) ? N / 32 + (pt >> 1) : (pt >> 1);
  return pt;
}
__host__ __device__ inline size_t weight_offset(int dtype, int layout, int K, int N, int k, int n) {
  const int pt = packed_tile_of(layout, N, n >> 4);
  const int r = n & 15;
  if (dtype == FRT_BF16) {
    const int ks = k >> 5, kk = k & 31;
    const int lane = r + 16 * (kk >> 3);
    return ((size_t)pt * (K >> 5) + ks) * 1024 + (size_t)lane * 16 + (size_t)(kk & 7) * 2;
  }
  const int ks = k >> 7, kk = k & 127;
  const int lane = r + 16 * ((kk >> 4) & 3);
  const int half = kk >> 6;
  return ((size_t)pt * (K >> 7) + ks) * 2048 + (size_t)half * 1024 + (size_t)lane * 16 + (kk & 15);
}

// Packed MXFP4 weight: 1088-byte tiles in the same (pt, ks) order.  Lane L of a tile
// holds column n = 16*lt + L%16 and the OCP MX block g = L/16 of the k-step, k = ks*128 +
// 32g + q for q = 0..31: FP4 code q in byte L*16 + q/2 (even q in the low nibble), its
// E8M0 scale byte at 1024 + L.  This is the operand order the FP4 x FP8 MFMA pairs with
// the e4m3 activation order above, and one lane's scale covers exactly its own block.
__host__ __device__ inline size_t mx_tile_offset(int layout, int K, int N, int k, int n) {
  return ((size_t)packed_tile_of(layout, N, n >> 4) * (K >> 7) + (k >> 7)) * 1088;
}
__host__ __device__ inline size_t mx_code_byte(int layout, int K, int N, int k, int n) {
  const int lane = (n & 15) + 16 * ((k >> 5) & 3);
  return mx_tile_offset(layout, K, N, k, n) + (size_t)lane * 16 + ((k & 31) >> 1);
}
__host__ __device__ inline size_t mx_scale_byte(int layout, int K, int N, int k, int n) {
  const int lane = (n & 15) + 16 * ((k >> 5) & 3);
  return mx_tile_offset(layout, K, N, k, n) + 1024 + lane;
}

// ------------------------------------------------------------------ number formats (device)
// float -> bfloat16 bits, round to nearest even; NaN -> canonical quiet NaN.
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u | ((u >> 16) & 0x8000u);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
  return __builtin_bit_cast(float, (b & 0xffffu) << 16);
}
// float -> OCP E4M3FN code: clamp to +-448 first (the hardware convert rounds to
// nearest even but turns magnitudes past the format into NaN), NaN -> 0x7F.
__device__ __forceinline__ uint32_t e4m3_code(float f) {
  if (f != f) return 0x7fu;
  const float c = fminf(fmaxf(f, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xffu;
}
// Four e4m3 codes packed little-endian into one dword.
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  const bool nan = (a != a) || (b != b) || (c != c) || (d != d);
  if (!nan) {
    const float lo = 448.0f, nlo = -448.0f;
    int v = __builtin_amdgcn_cvt_pk_fp8_f32(fminf(fmaxf(a, nlo), lo), fminf(fmaxf(b, nlo), lo), 0, false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32(fminf(fmaxf(c, nlo), lo), fminf(fmaxf(d, nlo), lo), v, true);
    return (uint32_t)v;
  }
  return e4m3_code(a) | (e4m3_code(b) << 8) | (e4m3_code(c) << 16) | (e4m3_code(d) << 24);
}
// Two values to bf16 with the gfx950 convert (round to nearest even; matches bf16_bits on
// every non-NaN input).
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
typedef float f32x2_hw __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16_pack2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_hw){a, b}, bf16x2_hw));
}

// Single rounding of a float64 value whose float32 rounding may land exactly on a
// rounding boundary of the narrow format although the float64 value does not (double
// rounding): in that case step the float32 value one ulp towards the float64 one, so the
// narrow format's round-to-nearest-even sees the side the exact value is on.
__device__ __forceinline__ float toward(float f, double exact) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  const bool away = (double)f < exact ? f >= 0.f : f <= 0.f;  // magnitude grows
  return __builtin_bit_cast(float, away ? u + 1u : u - 1u);
}
// bf16 code of a float64 value, rounded once (weights folded with gamma).
__device__ __forceinline__ uint32_t bf16_bits_exact(double x) {
  float f = (float)x;
  if ((__builtin_bit_cast(uint32_t, f) & 0xffffu) == 0x8000u && (double)f != x) f = toward(f, x);
  return bf16_bits(f);
}
// E4M3 code of a float64 value, rounded once: boundaries sit at 4 bits of significand in
// the normal range (|v| >= 2^-6) and at odd multiples of 2^-10 below it.
__device__ __forceinline__ uint32_t e4m3_code_exact(double x) {
  float f = (float)x;
  const float a = fabsf(f);
  if ((double)f != x && a < 448.0f) {
    bool mid;
    if (a >= 0.015625f) {
      mid = (__builtin_bit_cast(uint32_t, a) & 0xfffffu) == 0x80000u;
    } else {
      const float t = a * 512.0f;  // exact
      mid = t - floorf(t) == 0.5f;
    }
    if (mid) f = toward(f, x);
  }
  return e4m3_code(f);
}

// Write 4 consecutive logical k (k % 4 == 0) of row m of a packed operand.
// e4m3 values are divided by the static activation scale first (correctly rounded).
__device__ __forceinline__ void store_operand4(uint8_t* op, int dtype, int MB, int m, int k, float v0,
                                               float v1, float v2, float v3, float scale_e4m3,
                                               bool zero) {
  const size_t off = operand_offset(dtype, MB, m, k);
  if (dtype == FRT_BF16) {
    u32x2 w;
    w.x = zero ? 0u : bf16_pack2(v0, v1);
    w.y = zero ? 0u : bf16_pack2(v2, v3);
    *reinterpret_cast<u32x2*>(op + off) = w;
  } else {
    uint32_t w = zero ? 0u : e4m3_pack4(v0 / scale_e4m3, v1 / scale_e4m3, v2 / scale_e4m3, v3 / scale_e4m3);
    *reinterpret_cast<uint32_t*>(op + off) = w;
  }
}

__device__ __forceinline__ float load_scale(const float* p, float v) { return p ? __ldg(p) : v; }

// Calibration: fold |values| into a device-wide running maximum.  Non-negative floats
// order like their bit patterns, so an unsigned atomic max is exact and order-free.
__device__ __forceinline__ void record_amax(unsigned* amax, float a0, float a1, float a2, float a3) {
  if (!amax) return;
  const float m = fmaxf(fmaxf(fabsf(a0), fabsf(a1)), fmaxf(fabsf(a2), fabsf(a3)));
  if (m > 0.f) atomicMax(amax, __builtin_bit_cast(unsigned, m));
}

// Four consecutive columns n0..n0+3 of row m of a fused QKV output, rounded to bf16 and
// written where attention reads them (the section boundaries are multiples of 16):
// Q row-major [m][nq], K row-major [m][hd], V transposed v_out[d * v_ld + m].
__device__ __forceinline__ void store_qkv4(uint16_t* q_out, uint16_t* k_out, uint16_t* v_out, int nq, int hd,
                                           int v_ld, int m, int n0, f32x4 c) {
  if (n0 < nq + hd) {
    uint16_t* dst = n0 < nq ? q_out + (size_t)m * nq + n0 : k_out + (size_t)m * hd + (n0 - nq);
    u32x2 w;
    w.x = bf16_pack2(c.x, c.y);
    w.y = bf16_pack2(c.z, c.w);
    *reinterpret_cast<u32x2*>(dst) = w;
  } else {
    uint16_t* dst = v_out + (size_t)(n0 - nq - hd) * v_ld + m;
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[(size_t)r * v_ld] = (uint16_t)bf16_bits(c[r]);
  }
}

// ------------------------------------------------------------------ cross-lane butterflies
// One step of an xor butterfly over a 64-lane wave: v combined with the value of lane
// (lane ^ OFF), on the VALU instead of the LDS permute path of __shfl_xor.  OFF = 16 and
// 32 use the gfx950 lane swaps, which return the value pair (own, partner) in a
// row-dependent order; OFF = 1, 2, 8 are one DPP move (quad permutes, a row rotation by
// 8) and OFF = 4 is two (the half-row mirror, then a quad reversal).  Addition and
// maximum are commutative, so every lane gets bitwise what v + __shfl_xor(v, OFF) (or
// fmaxf) gives it.  All 64 lanes must be active.
template <int OFF>
__device__ __forceinline__ float xor_partner_dpp(float v) {
  const int x = __float_as_int(v);
  if constexpr (OFF == 1) return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false));
  else if constexpr (OFF == 2) return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false));
  else if constexpr (OFF == 8) return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false));
  else {
    static_assert(OFF == 4, "DPP partner for OFF in {1, 2, 4, 8}");
    const int m = __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false);  // lane 7 - i within 8
    return __int_as_float(__builtin_amdgcn_update_dpp(0, m, 0x1B, 0xF, 0xF, false));  // then 3 - j within 4
  }
}
template <int OFF>
__device__ __forceinline__ float xor_add(float v) {
  if constexpr (OFF == 16 || OFF == 32) {
    const unsigned u = __float_as_uint(v);
    const auto r = OFF == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                             : __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    return v + xor_partner_dpp<OFF>(v);
  }
}
template <int OFF>
__device__ __forceinline__ float xor_max(float v) {
  if constexpr (OFF == 16 || OFF == 32) {
    const unsigned u = __float_as_uint(v);
    const auto r = OFF == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                             : __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  } else {
    return fmaxf(v, xor_partner_dpp<OFF>(v));
  }
}

// ------------------------------------------------------------------ weight touching
// The packed weight bytes a following GEMM launch will read, described by that launch's
// shape, so that a latency-bound kernel can read them ahead from workgroups on the same
// XCDs as the GEMM workgroups that will stream them (their L2 then serves the GEMM; the
// memory-side cache serves it otherwise).  Workgroups are dispatched round-robin over the
// 8 XCDs, so linear workgroup id L runs on XCD L % 8.
struct WeightTouch {
  const uint8_t* w;          // null: nothing to touch
  int tb, ks;                // tile bytes; k-steps of the whole K
  int nt, kps, col_groups, row_groups, splits;
  int part, parts;           // touch units u with u % parts == part
};

// Reads one dword of every 64-byte segment of the GEMM workgroups' weight bytes that
// belong to this workgroup's XCD, spread over the touching workgroups of that XCD among
// the `count` with linear ids [first, first + count).  Returns a value the caller folds
// into a store that never happens, so the loads stay.
__device__ __forceinline__ unsigned touch_weights(const WeightTouch& t, int L, int first, int count) {
  if (!t.w) return 0u;
  const int c = L & 7;
  const int c0 = (c - (first & 7) + 8) & 7;     // offset of XCD c's first toucher
  const int i = (L - first - c0) >> 3;           // index among them
  const int nc = (count - c0 + 7) >> 3;          // how many there are
  const int per_xcd = t.row_groups > 1 ? ((t.col_groups - c + 7) >> 3) * t.splits
                                       : (t.col_groups * t.splits - c + 7) >> 3;
  const int nunits = per_xcd > 0 ? per_xcd : 0;
  const int nseg = t.kps * t.tb / 64;  // per tile
  // One flat range of (selected unit, tile, segment) over the XCD's touchers, 4 loads per
  // thread and round: every toucher pays one memory round trip per 4 * nc * blockDim
  // segments, however the bytes fall into units.  (A loop over whole units cost a round
  // trip per unit: 12 of the second producer's 20 touchers per XCD had two.  Measured on
  // MI355X, paired: -0.20 / -0.25 us per layer at M=50 / M=10 bf16, -0.17 e4m3.)
  const int nsel = nunits > t.part ? (nunits - t.part + t.parts - 1) / t.parts : 0;
  const int per_unit = t.nt * nseg;
  const int total = nsel * per_unit;
  unsigned acc = 0u;
  for (int f0 = i * blockDim.x + threadIdx.x; f0 < total; f0 += 4 * nc * blockDim.x) {
    unsigned v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int f = f0 + q * nc * blockDim.x;
      v[q] = 0u;
      if (f < total) {
        const int j = f / per_unit, r = f - j * per_unit, tt = r / nseg, sg = r - tt * nseg;
        const int u = t.part + j * t.parts;
        int g, y;
        if (t.row_groups > 1) {
          g = c + 8 * (u / t.splits);
          y = u % t.splits;
        } else {
          const int Lg = c + 8 * u;
          g = Lg % t.col_groups;
          y = Lg / t.col_groups;
        }
        v[q] = *reinterpret_cast<const unsigned*>(t.w + ((size_t)(g * t.nt + tt) * t.ks + (size_t)y * t.kps) * t.tb +
                                                    (size_t)sg * 64);
      }
    }
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  return acc;
}

// ------------------------------------------------------------------ kernel parameter blocks
struct RnqParams {
  int M, K, MB;
  const float* x;            // [splits][M][K] or null
  int x_splits;
  float x_scale;
  const float* x_scale_ptr;  // device scalar overriding x_scale (chain), or null
  const float* x_colscale;   // [K] or null
  const float* residual;     // [M][K]
  float* residual_out;       // [M][K] or null
  const float* gate;         // [K] or null
  const float* ada_scale;    // [K] or null
  const float* ada_shift;    // [K] or null
  float eps;
  int out_dtype;
  float act_scale;
  const float* act_scale_ptr;
  uint8_t* operand;          // packed or null
  unsigned* amax;            // calibration: running max |value before rounding| (float bits), or null
  WeightTouch touch;         // weights of a following GEMM read ahead by extra workgroups
  int touch_wgs;             // extra workgroups after the rows (a multiple of 8), or 0
  unsigned* sink;            // never written in practice (keeps the touch loads)
};

struct GemmParams {
  int M, N, K, MB, splits;
  int ab_dtype, layout;
  int ksteps_per_split;      // K / kstep / splits
  // set at launch from the tile shape (so the kernel does no integer division):
  int kwaves;                // waves per workgroup splitting the chunk
  int run;                   // k-steps per wave (ksteps_per_split / kwaves)
  int ksteps;                // k-steps of the whole K
  int row_groups, col_groups;  // workgroup grid per split
  const uint8_t* a;
  const uint8_t* w;
  const float* colscale;
  float act_scale;
  const float* act_scale_ptr;
  float* partials;           // [splits][M][N] when epi == NONE or splits > 1
  int epi;                   // epilogue applied in-kernel (only with splits == 1)
  void* out;
  int out_dtype;
  float out_scale;
  const float* out_scale_ptr;
  // kEpiQkv: columns [0, nq) -> q_out[m][.], [nq, nq+hd) -> k_out[m][.], then V^T
  uint16_t* q_out;
  uint16_t* k_out;
  uint16_t* v_out;
  int nq, hd, v_ld;
  unsigned* amax;            // calibration of the SiLU-gate output, or null
};

struct ReduceParams {
  int M, N, MB, splits;
  const float* partials;
  float act_scale;
  const float* act_scale_ptr;
  const float* colscale;
  int epi;
  void* out;
  int out_dtype;
  float out_scale;
  const float* out_scale_ptr;
  uint16_t* q_out;
  uint16_t* k_out;
  uint16_t* v_out;
  int nq, hd, v_ld;
  unsigned* amax;
};

struct AttnParams {
  int M, MB, n_heads, kv_len;
  const uint16_t* q;         // [M][n_heads*128] bf16
  const uint16_t* k;         // [kv_len][128] bf16 (prefix rows, then the M own rows)
  const uint16_t* vt;        // [128][ldv] bf16, V transposed (key index contiguous)
  int ldv;                   // >= kv_len rounded up to 32
  int chunk_keys;            // keys per workgroup (set by the launcher)
  int out_dtype;
  float out_scale;
  const float* out_scale_ptr;
  uint8_t* operand;
  float* workspace;          // chunk partial records when the key axis is split
  unsigned* amax;            // calibration of the attention output, or null
};

// Epilogue codes used inside the library beyond the public frt_epilogue values.
constexpr int kEpiQkv = 4;   // reduce + scale recovery + bf16, scattered into Q / K / V rows

size_t attention_workspace_bytes(int M, int n_heads, int kv_len);
int attention_kernel_count(int M, int n_heads, int kv_len);
bool attention_oproj_fusable(int M, int n_heads, int kv_len, int N);

// Launchers (stream-ordered, no validation: callers validate first).
hipError_t launch_rnq(const RnqParams& p, hipStream_t s);
hipError_t launch_gemm(const GemmParams& p, hipStream_t s);
// What launch_gemm(p) will read of p.w, as touch units; split into `parts` parts.
WeightTouch gemm_weight_touch(const GemmParams& p, int part, int parts);
hipError_t launch_reduce(const ReduceParams& p, hipStream_t s);
// attention key chunks, then their merge fused with the O projection (one split per head)
hipError_t launch_attention_oproj(const AttnParams& p, const GemmParams& o_proj, hipStream_t s);
hipError_t launch_attention(const AttnParams& p, hipStream_t s);
// Library choices of split count and waves per workgroup.
int choose_splits(int M, int N, int K, int dtype, int epi);

}  // namespace frt
