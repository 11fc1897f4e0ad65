// Skinny split-K GEMM kernel template (instantiated per weight format and epilogue in the
// gemm_{bf16,e4m3,mxfp4}{,_silu}.hip translation units; host side in gemm.hip).
//
// Pages: observation-age notes ("思考探索：具身推理加速，先看动作执行时观测有多旧"),
// section "小 M GEMM 要看并行度，也要看归约代价" (C = A W with few rows, cut along K into
// FP32 partial products that a consumer reduces), section "静态量化改变了两次矩阵乘之间的工作"
// (the GEMM's scale recovery remains after static quantisation).
//
// Mapping (gfx950): the weight tile is the MFMA's A operand (16 output columns x one
// k-step) and the activation tile its B operand (one k-step x 16 action rows), so the
// 16x16 accumulator holds C^T for 16 columns x 16 rows and M (<= 64) occupies 1..4
// column blocks.  Weights are pre-packed so that one 16-byte load per lane is one tile
// (1 KB per wave load, fully coalesced, straight into VGPRs with no LDS round trip);
// activations come packed the same way from the producer.
//
// Every launch starts with a cold instruction cache, so each kernel carries only the
// code of its own epilogue (a template parameter): a long branchy tail costs fetch
// latency on every launch.
#pragma once
#include <type_traits>
#include "frt_internal.hpp"

namespace frt {

enum GemmEpi { kGemmPartial = 0, kGemmStore = 1, kGemmSiluBf16 = 2, kGemmSiluE4m3 = 3, kGemmQkv = 4 };

// Tile shape of a launch: NT column tiles and MB row blocks per workgroup, kw waves with
// PER k-steps per round; (col_groups x row_groups) workgroups per split.  `fast` selects
// a kernel specialised for the common cases: kFastShape = four waves with one round each;
// kFastPlain = that and no scale read through a pointer (no column scales, no calibration
// maxima).
enum GemmFast { kGeneric = 0, kFastShape = 1, kFastPlain = 2 };
struct GemmShape {
  int nt, mbw, per, kw, col_groups, row_groups, epi;
  int fast;
};

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
template <>
struct Frag<FRT_MXFP4> {
  u32x4 v;     // 32 FP4 codes: one OCP MX block
  unsigned s;  // its E8M0 scale byte
};

// Word 3 of a gfx9 buffer resource: 32-bit data format, no swizzle, raw (stride 0)
// addressing; loads at offsets >= the resource's byte count return zeros.
constexpr int kBufferWord3 = 0x00020000;

// VGPRs a fragment holds per lane (the register budget of a round's loads).
constexpr int frag_regs(int dt) { return dt == FRT_BF16 ? 4 : (dt == FRT_MXFP4 ? 5 : 8); }

// One MFMA operand tile per wave: 16 bytes per lane (bf16), two 16-byte halves (e4m3),
// or 16 bytes of FP4 codes plus the lane's scale byte (MXFP4).
// STREAM marks weight loads non-temporal so the single-use weight stream does not evict
// the activation tiles every workgroup re-reads from L2.  (A compile-time choice: two
// loads of one address behind a run-time select get merged and lose the hint.)
template <int DT, bool STREAM>
__device__ __forceinline__ void load_frag(Frag<DT>& f, const uint8_t* tile, int lane) {
  const u32x4* p0 = reinterpret_cast<const u32x4*>(tile + lane * 16);
  if constexpr (DT == FRT_BF16) {
    if constexpr (STREAM) f.v = __builtin_nontemporal_load(p0);
    else f.v = *p0;
  } else if constexpr (DT == FRT_MXFP4) {
    static_assert(STREAM, "MXFP4 is a weight format");
    f.v = __builtin_nontemporal_load(p0);
    f.s = __builtin_nontemporal_load(tile + 1024 + lane);
  } else {
    const u32x4* p1 = reinterpret_cast<const u32x4*>(tile + 1024 + lane * 16);
    if constexpr (STREAM) {
      f.v0 = __builtin_nontemporal_load(p0);
      f.v1 = __builtin_nontemporal_load(p1);
    } else {
      f.v0 = *p0;
      f.v1 = *p1;
    }
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
// e4m3 x e4m3 with exact products: a lane's 32 codes of the 128-wide k-step are four groups
// of 8, each decoded to bf16 (every e4m3 value is a bf16 value, so the decode is exact) and
// multiplied by a bf16 MFMA, whose products are exact and whose sums are fp32.  Weights
// and activations take the same groups, so the four MFMAs add each of the 128 products
// once.  The fp8 MFMA above keeps about 13 bits of its internal sum: against the float64
// oracle its partial sums are off by about 1.5e-5 (relative), and through flipped e4m3
// codes the SiLU output of the M=10 FP8 block (AdaRMSNorm -> QKV, gate|up + SiLU, down)
// by 2.6e-3, over the 2e-3 its precision allows; exact, 4.5e-8 and 0.
// Kernels take this form when M <= 16, where every workgroup holds one 16-row block and
// the extra MFMAs and conversions are cheap: measured on MI355X (paired), +0.40 us per
// layer of the e4m3 chain at M=10.  With four row blocks they are not: at M=50 the chain
// lost 0.72 us per layer and the K=2048, N=16384 gate|up GEMM went from 9.8 to 12.9 us,
// so M > 16 keeps the fp8 MFMA.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo4, uint32_t hi4) {
  const u32x4 r = {e4m3x2_to_bf16x2<false>(lo4), e4m3x2_to_bf16x2<true>(lo4), e4m3x2_to_bf16x2<false>(hi4),
                   e4m3x2_to_bf16x2<true>(hi4)};
  return __builtin_bit_cast(bf16x8, r);
}
__device__ __forceinline__ f32x4 mma_exact(const Frag<FRT_E4M3>& w, const Frag<FRT_E4M3>& a, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(w.v0.x, w.v0.y), e4m3x8_to_bf16(a.v0.x, a.v0.y), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(w.v0.z, w.v0.w), e4m3x8_to_bf16(a.v0.z, a.v0.w), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(w.v1.x, w.v1.y), e4m3x8_to_bf16(a.v1.x, a.v1.y), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(w.v1.z, w.v1.w), e4m3x8_to_bf16(a.v1.z, a.v1.w), c, 0, 0, 0);
  return c;
}
// EXACT selects mma_exact (e4m3 weights and activations only)
template <bool EXACT, int WDT, int ADT>
__device__ __forceinline__ f32x4 mma_sel(const Frag<WDT>& w, const Frag<ADT>& a, f32x4 c) {
  if constexpr (EXACT) return mma_exact(w, a, c);
  else return mma(w, a, c);
}
// e4m3 x e4m3 products are exact when M <= 16 (the row count of the whole GEMM)
inline bool e4m3_exact(int M) { return M <= 16; }
__device__ __forceinline__ f32x4 mma(const Frag<FRT_MXFP4>& w, const Frag<FRT_E4M3>& a, f32x4 c) {
  i32x8 wa, aa;
  wa[0] = (int)w.v.x; wa[1] = (int)w.v.y; wa[2] = (int)w.v.z; wa[3] = (int)w.v.w;
  wa[4] = 0; wa[5] = 0; wa[6] = 0; wa[7] = 0;  // an FP4 operand is four dwords
  aa[0] = (int)a.v0.x; aa[1] = (int)a.v0.y; aa[2] = (int)a.v0.z; aa[3] = (int)a.v0.w;
  aa[4] = (int)a.v1.x; aa[5] = (int)a.v1.y; aa[6] = (int)a.v1.z; aa[7] = (int)a.v1.w;
  // format 4 = FP4 E2M1 weights under the lane's own E8M0 block scale, format 0 = e4m3
  // activations unscaled (their static scale is applied after the sum)
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wa, aa, c, 4, 0, 0, (int)w.s, 0, 127);
}

// SiLU(g) = g / (1 + e^-g) from the hardware exp2 and reciprocal (a few ulp; the parity
// tie band is 2^-17 of the summands).
__device__ __forceinline__ float silu_f(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f));
}

// Workgroup = (column-tile group g, row group r, K-chunk `split`).  Its kw waves split the
// chunk's k-steps into contiguous runs of PER * rounds; a wave issues its first PER
// k-steps' weight and activation loads before its first wait (a scheduling barrier keeps
// the compiler from interleaving them with the MFMAs, which would put a memory round trip
// between every few MFMAs), then, with more rounds, reloads each k-step slot with the next
// round's k-step right after that slot's MFMAs (a rolling pipeline).  The waves' sums are
// added in LDS in wave order, so results are bitwise deterministic and independent of
// the row grouping.  Row groups (XCD-aware: the groups that share a column group are
// eight workgroup ids apart, so they run on one XCD and its L2 serves the weight tile
// to all of them after one HBM read) spread GEMMs with few column tiles over more CUs.
// FAST (GemmFast) fixes four waves and a single round, and with kFastPlain drops the
// pointer-read scales: measured on MI355X, the shorter, branch-free code saves 0.4 us per
// launch of the gate|up GEMM.
template <int DT, int MB, int NT, int PER, int EPI, int FAST, bool PAD, bool EXACT = false>
__global__ void __launch_bounds__(256) skinny_gemm_kernel(const GemmParams p) {
  constexpr bool SHAPE = FAST != kGeneric, PLAIN = FAST == kFastPlain;
  constexpr int ADT = act_dtype_of(DT);   // operand (activation) format
  constexpr int TBW = tile_bytes_of(DT);  // weight tile bytes
  constexpr int TB = tile_bytes_of(ADT);  // operand tile bytes
  constexpr int NF = NT * MB;
  extern __shared__ f32x4 red[];  // [kwaves][NF][64]

  const int lane = threadIdx.x & 63;
  // wave index made provably uniform: MFMAs ignore EXEC, so every branch around them must
  // be a scalar branch, never an EXEC-masked one
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kw = SHAPE ? 4 : p.kwaves;
  const int KS = p.ksteps;
  const int run = p.run;  // = PER * rounds
  // grid: (col_groups, 1, splits), or with row groups (8 * row_groups, ceil(col_groups / 8),
  // splits), where x = 8 r + g % 8 and y = g / 8: linear id = g % 8 (mod 8), so all row
  // groups of a column group run on its XCD
  const int g_grid = p.row_groups == 1 ? (int)blockIdx.x : (int)(blockIdx.y * 8 + (blockIdx.x & 7));
  const int r = p.row_groups == 1 ? 0 : (int)(blockIdx.x >> 3);
  // padding workgroups of the row-group grid repeat the last column group's loads (in
  // bounds) and store nothing: no branch ahead of the loads, so every kernel argument is
  // fetched in one batch
  const bool active = g_grid < p.col_groups;
  const int g = active ? g_grid : p.col_groups - 1;
  const int mb0 = r * MB;  // first 16-row block of this workgroup
  const int split = blockIdx.z;
  const int ks_begin = split * p.ksteps_per_split + wave * run;

  const uint8_t* wbase[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) wbase[t] = p.w + (size_t)(g * NT + t) * KS * TBW;
  const uint8_t* abase = p.a + (size_t)mb0 * TB;
  const size_t astep = (size_t)p.MB * TB;

  f32x4 acc[NT][MB];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int b = 0; b < MB; ++b) acc[t][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // PER k-step slots of weight and activation fragments; slot u first holds k-step
  // ks_begin + u.  run = PER * rounds, rounds >= 1.
  Frag<DT> wf[PER][NT];
  Frag<ADT> af[PER][MB];
  // PAD kernels (M not a multiple of 16, single-round shapes): the lanes of the padding
  // rows of the last 16-row block (M = 50: 14 of 16) load nothing, since their columns of
  // the product are never stored.  bf16 operands skip them under EXEC; e4m3 operands read
  // the tile through a buffer resource that ends at the tile, with those lanes addressed
  // past its end (zeros, no memory access; an EXEC-masked e4m3 load made the compiler copy
  // a loaded register inside the masked block and wait there for every load in flight).
  // Measured on MI355X (paired on one box, bitwise equal outputs): bf16 chain 29.58 ->
  // 29.11 us/layer at M=50, 26.31 -> 25.37 at M=10; e4m3 26.84 -> 26.66 at M=50; MXFP4
  // weights 25.63 -> 25.47.  It is a compile-time variant: a run-time test around the
  // masked loads made kernels wait for more loads before their first MFMA, masked or not
  // (the K=2048 sweep's two-round bf16 GEMM at M=64: 16.3 -> 17.6 us; e4m3 at M=32: 8.3 ->
  // 8.6 us), and cost 0.8 us per layer of the M=10 bf16 chain.  bf16 through the buffer
  // resource instead of EXEC: 29.44 at M=50.
  const int rem_last = p.M - (mb0 + MB - 1) * 16;  // real rows of the last block (>= 16: full)
  const bool lane_row_live = (lane & 15) < rem_last;
  const int voff = lane_row_live ? lane * 16 : TB;
  auto load_slot = [&](int u, int ks) {
#pragma unroll
    for (int t = 0; t < NT; ++t) load_frag<DT, true>(wf[u][t], wbase[t] + (size_t)ks * TBW, lane);
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      const uint8_t* at = abase + (size_t)ks * astep + (size_t)b * TB;
      if (PAD && b == MB - 1) {
        if constexpr (ADT == FRT_BF16) {
          af[u][b] = Frag<ADT>{};
          if (lane_row_live) load_frag<ADT, false>(af[u][b], at, lane);
        } else {
          const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)at, (short)0, TB, kBufferWord3);
          af[u][b].v0 = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, 0);
          af[u][b].v1 = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 1024, 0, 0);
        }
      } else {
        load_frag<ADT, false>(af[u][b], at, lane);
      }
    }
  };

  auto mma_slot = [&](int u) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int b = 0; b < MB; ++b) acc[t][b] = mma_sel<EXACT>(wf[u][t], af[u][b], acc[t][b]);
  };
  // With e4m3 weights the epilogue's scales are requested ahead of the k-step loads:
  // after the sums, the scalar scale loads and the column-scale loads each cost a memory
  // round trip.  Measured on MI355X (paired, bitwise equal outputs): e4m3 chain 26.38 ->
  // 26.03 us/layer at M=50, 23.55 -> 23.20 at M=10.  (The same for MXFP4 weights, which
  // carry no column scales, lost 0.13 us; they keep the scalar loads in the epilogue.)
  constexpr bool SILU = EPI == kGemmSiluBf16 || EPI == kGemmSiluE4m3;
  constexpr bool SCALED = EPI != kGemmPartial && !PLAIN && DT == FRT_E4M3;
  constexpr int NCS = SILU ? (NT / 2 > 0 ? NT / 2 : 1) : NT;
  float as = p.act_scale, os = p.out_scale;
  f32x4 csa[NCS], csb[NCS];  // column scales of this lane's 4 columns (SiLU: gate, up)
  if constexpr (SCALED) {
    as = load_scale(p.act_scale_ptr, p.act_scale);
    if constexpr (SILU) os = load_scale(p.out_scale_ptr, p.out_scale);
#pragma unroll
    for (int t = 0; t < NCS; ++t) {
      csa[t] = f32x4{1.f, 1.f, 1.f, 1.f};
      csb[t] = f32x4{1.f, 1.f, 1.f, 1.f};
    }
    if (p.colscale) {
#pragma unroll
      for (int t = 0; t < NCS; ++t) {
        if constexpr (SILU) {
          const int ng = ((g * NT) / 2 + t) * 16 + 4 * (lane >> 4);
          csa[t] = *reinterpret_cast<const f32x4*>(p.colscale + ng);
          csb[t] = *reinterpret_cast<const f32x4*>(p.colscale + ng + p.N / 2);
        } else {
          csa[t] = *reinterpret_cast<const f32x4*>(p.colscale + logical_tile_of(p.layout, p.N, g * NT + t) * 16 +
                                                   4 * (lane >> 4));
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) load_slot(u, ks_begin + u);
  __builtin_amdgcn_sched_barrier(0);
  // The Q/K/V scatter's pointers and sizes share no kernel-argument cache line with what
  // the loads use.  Requested here (the empty asm only makes them live), their scalar
  // round trip overlaps the loads in flight; read at their first use, it came after the
  // MFMAs, at the very end of the kernel.  (Requested before the loads, together with
  // the fused merge's arguments at its kernel start, the MXFP4-weight chain at M=50 ran
  // 0.1-0.25 us per layer slower than with both after the loads.)
  if constexpr (EPI == kGemmQkv) {
    asm volatile("" ::"s"(p.q_out), "s"(p.k_out), "s"(p.v_out), "s"(p.nq), "s"(p.hd), "s"(p.v_ld));
  }
  if constexpr (!SHAPE) {
    // Rolling pipeline over the further rounds: as soon as slot u's MFMAs have read it,
    // the slot is reloaded with the same slot of the next round, so a full round of loads
    // stays in flight instead of each round waiting for the last one's data and sums.
    const int rounds = run / PER;
    for (int r = 1; r < rounds; ++r) {
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        mma_slot(u);
        load_slot(u, ks_begin + r * PER + u);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) mma_slot(u);  // the last (or only) round
  if (!active) return;  // whole workgroup

  // ---- epilogue (one per kernel)
  if constexpr (!SCALED && !PLAIN && EPI != kGemmPartial) {
    as = load_scale(p.act_scale_ptr, p.act_scale);
    if constexpr (SILU) os = load_scale(p.out_scale_ptr, p.out_scale);
  }
  // fragment (t, b) finished: partial store, or scale recovery + store / Q-K-V scatter
  auto finish = [&](int t, int b, f32x4 v) {
    const int n0 = logical_tile_of(p.layout, p.N, g * NT + t) * 16 + 4 * (lane >> 4);
    const int m = (mb0 + b) * 16 + (lane & 15);
    if (m >= p.M) return;
    if constexpr (EPI == kGemmPartial) {
      *reinterpret_cast<f32x4*>(p.partials + ((size_t)split * p.M + m) * p.N + n0) = v;
    } else {
      f32x4 c = v * as;
      if constexpr (SCALED) c *= csa[SILU ? 0 : t];
      else if (!PLAIN && p.colscale) c *= *reinterpret_cast<const f32x4*>(p.colscale + n0);
      if constexpr (EPI == kGemmQkv) {
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
  };
  // SiLU-gate epilogue: packed tiles 2i (gate) and 2i+1 (up) of this workgroup pair up;
  // padding rows of the output operand get zero codes
  auto finish_pair = [&](int tp, int b, f32x4 vg, f32x4 vu) {
    // the in-kernel SiLU epilogue runs only on FRT_W_GATE_UP weights: packed tiles 2i and
    // 2i+1 are gate tile i and up tile i
    const int ng = ((g * NT) / 2 + tp) * 16 + 4 * (lane >> 4);
    const int nu = ng + p.N / 2;
    const int m = (mb0 + b) * 16 + (lane & 15);
    f32x4 cg = vg * as, cu = vu * as;
    if constexpr (SCALED) {
      cg *= csa[tp];
      cu *= csb[tp];
    } else if (!PLAIN && p.colscale) {
      cg *= *reinterpret_cast<const f32x4*>(p.colscale + ng);
      cu *= *reinterpret_cast<const f32x4*>(p.colscale + nu);
    }
    float z[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) z[e] = silu_f(cg[e]) * cu[e];
    store_operand4(reinterpret_cast<uint8_t*>(p.out), EPI == kGemmSiluBf16 ? FRT_BF16 : FRT_E4M3, p.MB, m, ng,
                   z[0], z[1], z[2], z[3], os, m >= p.M);
    if (!PLAIN && m < p.M) record_amax(p.amax, z[0], z[1], z[2], z[3]);
  };

  // combine the kw (<= 4) waves' sums in wave order through LDS (with one wave too: a
  // loop over LDS is far shorter code than unrolling every fragment's epilogue)
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int b = 0; b < MB; ++b) red[((size_t)wave * NF + t * MB + b) * 64 + lane] = acc[t][b];
  __syncthreads();
  auto sum_waves = [&](int f) {
    f32x4 v = red[(size_t)f * 64 + lane];
#pragma unroll
    for (int w2 = 1; w2 < 4; ++w2)
      if (w2 < kw) v += red[((size_t)w2 * NF + f) * 64 + lane];
    return v;
  };
  if constexpr (EPI == kGemmSiluBf16 || EPI == kGemmSiluE4m3) {
    constexpr int NPAIR = (NT / 2) * MB;
    for (int f = wave; f < NPAIR; f += kw) {
      const int tp = f / MB, b = f % MB;
      finish_pair(tp, b, sum_waves((2 * tp) * MB + b), sum_waves((2 * tp + 1) * MB + b));
    }
  } else {
    for (int f = wave; f < NF; f += kw) finish(f / MB, f % MB, sum_waves(f));
  }
}

// ------------------------------------------------------------------ typed dispatch
template <int DT, int MB, int NT, int PER, int EPI>
static hipError_t launch_t(const GemmParams& p, const GemmShape& sh, hipStream_t s) {
  constexpr bool silu = EPI == kGemmSiluBf16 || EPI == kGemmSiluE4m3;
  if constexpr (PER * (NT * frag_regs(DT) + MB * frag_regs(act_dtype_of(DT))) > 192 || (silu && NT % 2)) {
    return hipErrorInvalidValue;  // never chosen (register budget / SiLU pairs): not instantiated
  } else {
    const dim3 grid = sh.row_groups == 1 ? dim3(sh.col_groups, 1, p.splits)
                                         : dim3(8 * sh.row_groups, (sh.col_groups + 7) / 8, p.splits);
    const size_t lds = (size_t)p.kwaves * NT * MB * 64 * sizeof(f32x4);
    const bool pad = p.M % 16 != 0;
    auto go = [&](auto exact) {
      constexpr bool X = decltype(exact)::value;
      if (sh.fast == kFastPlain && pad)
        hipLaunchKernelGGL((skinny_gemm_kernel<DT, MB, NT, PER, EPI, kFastPlain, true, X>), grid, dim3(256), lds, s, p);
      else if (sh.fast == kFastPlain)
        hipLaunchKernelGGL((skinny_gemm_kernel<DT, MB, NT, PER, EPI, kFastPlain, false, X>), grid, dim3(256), lds, s, p);
      else if (sh.fast == kFastShape && pad)
        hipLaunchKernelGGL((skinny_gemm_kernel<DT, MB, NT, PER, EPI, kFastShape, true, X>), grid, dim3(256), lds, s, p);
      else if (sh.fast == kFastShape)
        hipLaunchKernelGGL((skinny_gemm_kernel<DT, MB, NT, PER, EPI, kFastShape, false, X>), grid, dim3(256), lds, s, p);
      else
        hipLaunchKernelGGL((skinny_gemm_kernel<DT, MB, NT, PER, EPI, kGeneric, false, X>), grid, dim3(64 * p.kwaves), lds, s,
                           p);
    };
    if constexpr (DT == FRT_E4M3 && MB == 1) {
      if (e4m3_exact(p.M)) go(std::true_type{});
      else go(std::false_type{});
    } else {
      go(std::false_type{});
    }
    return hipGetLastError();
  }
}

template <int DT, int EPI, int MB, int NT>
static hipError_t launch_per(const GemmParams& p, const GemmShape& sh, hipStream_t s) {
  switch (sh.per) {
    case 1: return launch_t<DT, MB, NT, 1, EPI>(p, sh, s);
    case 2: return launch_t<DT, MB, NT, 2, EPI>(p, sh, s);
    case 4: return launch_t<DT, MB, NT, 4, EPI>(p, sh, s);
    default: return launch_t<DT, MB, NT, 8, EPI>(p, sh, s);
  }
}

template <int DT, int EPI, int MB>
static hipError_t launch_nt(const GemmParams& p, const GemmShape& sh, hipStream_t s) {
  switch (sh.nt) {
    case 1: return launch_per<DT, EPI, MB, 1>(p, sh, s);
    case 2: return launch_per<DT, EPI, MB, 2>(p, sh, s);
    default: return launch_per<DT, EPI, MB, 4>(p, sh, s);
  }
}

// All kernels of one (weight format, epilogue); explicitly instantiated in the gemm_*.hip
// translation units, a few per file, so that they compile in parallel.
template <int DT, int EPI>
hipError_t launch_gemm_epi(const GemmParams& p, const GemmShape& sh, hipStream_t s) {
  switch (sh.mbw) {
    case 1: return launch_nt<DT, EPI, 1>(p, sh, s);
    case 2: return launch_nt<DT, EPI, 2>(p, sh, s);
    case 3: return launch_nt<DT, EPI, 3>(p, sh, s);
    default: return launch_nt<DT, EPI, 4>(p, sh, s);
  }
}

}  // namespace frt
