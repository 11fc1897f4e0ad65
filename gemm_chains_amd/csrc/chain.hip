// The action-decoder layer chain: layers x flow steps of producer -> GEMM -> consumer
// kernels over persistent named buffers, captured once into a hipGraph and replayed.
//
// Pages: observation-age notes ("思考探索：具身推理加速，先看动作执行时观测有多旧"), section
// "CUDA Graph 与图化简分别省掉什么" (record the GPU work once, replay it with the same
// arguments and addresses, new inputs go into agreed buffers, static shapes), section
// "固定工作负载给了系统优化更多余地" (batch 1, fixed action length: fixed graph and
// preallocated buffers, kernels chosen for the real shapes), section
// "静态量化改变了两次矩阵乘之间的工作" (18 layers x 10 denoising steps = 180 passes; the
// consumer of layer l prepares layer l+1's input with layer l+1's conditioning);
// FlashRT-PAI abstract ("FlashRT-PAI: Fast Kernels Are Not Fast Pipelines for Physical AI
// Inference": named buffers that persist across decisions).
#include "frt_internal.hpp"

#include <string.h>
#include <new>
#include <vector>

namespace frt {

enum { SITE_QKV = 0, SITE_O = 1, SITE_UP = 2, SITE_DOWN = 3 };

enum { MOD_SCALE = 0, MOD_SHIFT = 1, MOD_GATE = 2 };

struct Buf {
  size_t off = 0, bytes = 0;
};

struct ChainLayout {
  int s_qkv = 0, s_o = 0, s_up = 0, s_down = 0;
  bool fuse_o = false;                                     // attention merge fused with the O projection
  int nqkv = 0, nattn = 0;
  int kv_len = 0;                                          // prefix + own rows
  int ldv = 0;                                             // V^T row length (kv_len padded to 32)
  size_t op_qkv = 0, op_o = 0, op_up = 0, op_down = 0;     // operand bytes
  size_t pq = 0, po = 0, pu = 0, pd = 0;                   // partial bytes (one copy)
  size_t qb = 0, attn_ws = 0;
  Buf x_in, x_out, mod, act, kc, vc, h, q, aws, sink, amax, a_qkv, a_o, a_up, a_down, p_qkv, p_o, p_up, p_down;
  Buf d_h_attn, d_h_mlp, d_a_qkv, d_a_o, d_a_up, d_a_down, d_p_o, d_p_down, d_q, d_k, d_v;
  size_t total = 0;
};

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

static int validate_desc(const frt_chain_desc* d) {
  FRT_CHECK(d, FRT_E_NULL);
  FRT_CHECK(d->layers >= 1 && d->layers <= 256 && d->steps >= 1 && d->steps <= 1000, FRT_E_SHAPE);
  FRT_CHECK(is_w_dtype(d->dtype), FRT_E_DTYPE);
  const int ks = kstep_of(d->dtype);
  FRT_CHECK(d->M >= 1 && d->M <= kMaxM, FRT_E_SHAPE);
  FRT_CHECK(d->hidden >= ks && d->hidden % ks == 0 && d->hidden <= kMaxProducerK, FRT_E_SHAPE);
  FRT_CHECK(d->head_dim == 128, FRT_E_SHAPE);
  FRT_CHECK(d->n_heads >= 1 && d->n_heads <= 16 && (d->n_heads * d->head_dim) % ks == 0, FRT_E_SHAPE);
  FRT_CHECK(d->prefix_len >= 0 && d->prefix_len <= 8192, FRT_E_SHAPE);
  FRT_CHECK(d->mlp >= ks && d->mlp % ks == 0 && d->mlp % 16 == 0, FRT_E_SHAPE);
  FRT_CHECK(d->eps >= 0.f && d->eps == d->eps, FRT_E_ARG);
  const int sp[4] = {d->splits_qkv, d->splits_o, d->splits_up, d->splits_down};
  for (int s : sp) FRT_CHECK(s == 0 || is_split(s), FRT_E_SPLITK);
  FRT_CHECK(d->w_qkv && d->w_o && d->w_up && d->w_down, FRT_E_NULL);
  for (int l = 0; l < d->layers; ++l) {
    FRT_CHECK(d->w_qkv[l] && d->w_o[l] && d->w_up[l] && d->w_down[l], FRT_E_NULL);
    FRT_CHECK(aligned16(d->w_qkv[l]) && aligned16(d->w_o[l]) && aligned16(d->w_up[l]) && aligned16(d->w_down[l]),
              FRT_E_ALIGN);
  }
  if (d->dtype == FRT_E4M3) {
    FRT_CHECK(d->s_qkv && d->s_o && d->s_up && d->s_down, FRT_E_NULL);
    for (int l = 0; l < d->layers; ++l) {
      FRT_CHECK(d->s_qkv[l] && d->s_o[l] && d->s_up[l] && d->s_down[l], FRT_E_NULL);
      FRT_CHECK(aligned16(d->s_qkv[l]) && aligned16(d->s_o[l]) && aligned16(d->s_up[l]) && aligned16(d->s_down[l]),
                FRT_E_ALIGN);
    }
  }
  return FRT_OK;
}

static int resolve_split(int s, int M, int N, int K, int dtype, int epi) {
  return s ? s : choose_splits(M, N, K, dtype, epi);
}

static int make_layout(const frt_chain_desc* d, ChainLayout& L) {
  const int M = d->M, H = d->hidden, F = d->mlp, dt = d->dtype;
  L.nqkv = (d->n_heads + 2) * d->head_dim;
  L.nattn = d->n_heads * d->head_dim;
  L.s_qkv = resolve_split(d->splits_qkv, M, L.nqkv, H, dt, kEpiQkv);
  L.s_o = resolve_split(d->splits_o, M, H, L.nattn, dt, FRT_EPI_NONE);
  // The attention merge runs inside the O projection when the key axis is split: that
  // projection then has one split per head.  Debug runs keep the two apart (so the
  // attention output can be inspected) with the same split, which makes them bitwise
  // equal to the fused chain.
  const int kv_len = d->prefix_len + M;
  if ((d->splits_o == 0 || d->splits_o == d->n_heads) && attention_oproj_fusable(M, d->n_heads, kv_len, H)) {
    L.s_o = d->n_heads;
    L.fuse_o = !d->keep_intermediates;
  }
  L.s_up = resolve_split(d->splits_up, M, 2 * F, H, dt, FRT_EPI_SILU_GATE_QUANT);
  L.s_down = resolve_split(d->splits_down, M, H, F, dt, FRT_EPI_NONE);
  const int ks = kstep_of(dt);
  FRT_CHECK((H / ks) % L.s_qkv == 0 && (L.nattn / ks) % L.s_o == 0 && (H / ks) % L.s_up == 0 &&
                (F / ks) % L.s_down == 0,
            FRT_E_SPLITK);
  const int adt = act_dtype_of(dt);  // GEMM operand format
  L.op_qkv = frt_operand_bytes(adt, M, H);
  L.op_o = frt_operand_bytes(adt, M, L.nattn);
  L.op_up = frt_operand_bytes(adt, M, H);
  L.op_down = frt_operand_bytes(adt, M, F);
  L.kv_len = d->prefix_len + M;
  L.ldv = (L.kv_len + 31) / 32 * 32;
  L.pq = L.s_qkv > 1 ? (size_t)L.s_qkv * M * L.nqkv * 4 : 0;
  L.qb = (size_t)M * L.nattn * 2;
  L.attn_ws = attention_workspace_bytes(M, d->n_heads, L.kv_len);
  L.po = (size_t)L.s_o * M * H * 4;
  L.pu = L.s_up > 1 ? (size_t)L.s_up * M * 2 * F * 4 : 0;
  L.pd = (size_t)L.s_down * M * H * 4;
  const size_t SL = (size_t)d->steps * d->layers;
  size_t off = 0;
  auto take = [&](Buf& b, size_t bytes) {
    b.off = off;
    b.bytes = bytes;
    off = align256(off + bytes);
  };
  take(L.x_in, (size_t)M * H * 4);
  take(L.x_out, (size_t)M * H * 4);
  take(L.mod, SL * 2 * 3 * H * 4);
  take(L.act, (size_t)d->layers * 4 * 4);
  take(L.kc, (size_t)d->layers * L.kv_len * d->head_dim * 2);
  take(L.vc, (size_t)d->layers * d->head_dim * L.ldv * 2);
  take(L.h, (size_t)M * H * 4);
  take(L.q, L.qb);
  take(L.aws, L.attn_ws);
  take(L.sink, 64);
  take(L.amax, (size_t)d->layers * 4 * 4);
  take(L.a_qkv, L.op_qkv);
  take(L.a_o, L.op_o);
  take(L.a_up, L.op_up);
  take(L.a_down, L.op_down);
  take(L.p_qkv, L.pq);
  take(L.p_o, L.po);
  take(L.p_up, L.pu);
  take(L.p_down, L.pd);
  if (d->keep_intermediates) {
    take(L.d_h_attn, SL * M * H * 4);
    take(L.d_h_mlp, SL * M * H * 4);
    take(L.d_a_qkv, SL * align256(L.op_qkv));
    take(L.d_a_o, SL * align256(L.op_o));
    take(L.d_a_up, SL * align256(L.op_up));
    take(L.d_a_down, SL * align256(L.op_down));
    take(L.d_p_o, SL * align256(L.po));
    take(L.d_p_down, SL * align256(L.pd));
    take(L.d_q, SL * align256(L.qb));
    take(L.d_k, SL * align256((size_t)M * d->head_dim * 2));
    take(L.d_v, SL * align256((size_t)M * d->head_dim * 2));
  }
  L.total = off;
  return FRT_OK;
}

}  // namespace frt

using namespace frt;

struct frt_chain {
  frt_chain_desc d;
  std::vector<const void*> wq, wo, wu, wd;
  std::vector<const float*> sq, so, su, sd;
  uint8_t* arena = nullptr;
  size_t arena_bytes = 0;
  ChainLayout L;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  int kernels = 0;
};

static uint8_t* at(frt_chain* c, const Buf& b, size_t idx = 0, size_t stride = 0) {
  return c->arena + b.off + idx * stride;
}

// Debug chains only: copy the own key rows [M][hd] of one layer's key cache and its own
// value columns of the transposed value cache ([hd][ldv], columns 0..M-1 from vt) into
// per-(step, layer) buffers, both row-major [M][hd], before the next flow step rewrites
// them.
__global__ void copy_own_kv_kernel(const uint16_t* __restrict__ k_own, const uint16_t* __restrict__ vt, int ldv,
                                   int M, int hd, uint16_t* __restrict__ k_dst, uint16_t* __restrict__ v_dst) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= M * hd) return;
  k_dst[i] = k_own[i];
  const int m = i / hd, e = i - m * hd;
  v_dst[i] = vt[(size_t)e * ldv + m];
}

// Enqueue the whole chain on `s` (eager launches; also what graph capture records).
// With prefetch_next, each producer reads the weights of a GEMM that follows it ahead,
// from extra workgroups on the XCDs that will stream them (the launch-overlap
// analogue), so that GEMM finds them in L2: the first producer the QKV weights, the
// second the down projection's.  Measured on MI355X (bf16, M=50): 31.8 -> 30.8 us/layer
// for the QKV placement on top of the down one.  Reading the gate|up weights in the
// attention kernels or the second producer slowed the chain (the extra traffic delays
// those kernels' own loads more than the GEMM gains).
static int enqueue_chain(frt_chain* c, hipStream_t s, int* count, unsigned* amax = nullptr) {
  const frt_chain_desc& d = c->d;
  const ChainLayout& L = c->L;
  const int M = d.M, H = d.hidden, F = d.mlp, MB = m_blocks(M);
  const bool e4 = d.dtype == FRT_E4M3;          // weights carry column scales
  const int adt = act_dtype_of(d.dtype);        // GEMM operand format
  const bool aq = adt == FRT_E4M3;              // operands carry static activation scales
  const bool dbg = d.keep_intermediates != 0;
  const size_t modsz = (size_t)3 * H;  // floats per (step, layer, sublayer)
  float* mod = (float*)at(c, L.mod);
  float* act = (float*)at(c, L.act);
  auto modp = [&](int k, int l, int sub, int row) { return mod + (((size_t)k * d.layers + l) * 2 + sub) * modsz + (size_t)row * H; };
  auto actp = [&](int l, int site) -> const float* { return aq ? act + l * 4 + site : nullptr; };
  int n = 0;
  const bool pf = d.prefetch_next != 0;
  unsigned* sink = (unsigned*)at(c, L.sink);
  const int rows = MB * 16;
  // read-ahead workgroups: on the CUs the rows leave free, at most 160 (paired on
  // MI355X: 128-160 beat the 192 / 240 that fill the free CUs by 0.03-0.15 us per layer
  // at M = 50 / 10; 64 or 96 lose 0.4-1.3 us, each toucher then reads too much)
  const int touch_wgs = ((256 - rows) / 8) * 8 < 160 ? ((256 - rows) / 8) * 8 : 160;

  const float* h_prev = (const float*)at(c, L.x_in);
  const float* pdown_prev = nullptr;
  int kp = -1, lp = -1;
  for (int k = 0; k < d.steps; ++k) {
    for (int l = 0; l < d.layers; ++l) {
      const size_t idx = (size_t)k * d.layers + l;
      float* h_attn = dbg ? (float*)at(c, L.d_h_attn, idx, (size_t)M * H * 4) : (float*)at(c, L.h);
      float* h_mlp = dbg ? (float*)at(c, L.d_h_mlp, idx, (size_t)M * H * 4) : (float*)at(c, L.h);
      uint8_t* a_qkv = dbg ? at(c, L.d_a_qkv, idx, align256(L.op_qkv)) : at(c, L.a_qkv);
      uint8_t* a_o = dbg ? at(c, L.d_a_o, idx, align256(L.op_o)) : at(c, L.a_o);
      uint8_t* a_up = dbg ? at(c, L.d_a_up, idx, align256(L.op_up)) : at(c, L.a_up);
      uint8_t* a_down = dbg ? at(c, L.d_a_down, idx, align256(L.op_down)) : at(c, L.a_down);
      float* p_qkv = (float*)at(c, L.p_qkv);
      float* p_o = dbg ? (float*)at(c, L.d_p_o, idx, align256(L.po)) : (float*)at(c, L.p_o);
      float* p_down = dbg ? (float*)at(c, L.d_p_down, idx, align256(L.pd)) : (float*)at(c, L.p_down);
      uint16_t* qbuf = dbg ? (uint16_t*)at(c, L.d_q, idx, align256(L.qb)) : (uint16_t*)at(c, L.q);
      uint16_t* kcl = (uint16_t*)at(c, L.kc) + (size_t)l * L.kv_len * d.head_dim;
      uint16_t* vcl = (uint16_t*)at(c, L.vc) + (size_t)l * d.head_dim * L.ldv;

      // the layer's four GEMMs
      GemmParams gq{};
      gq.M = M; gq.MB = MB; gq.ab_dtype = d.dtype; gq.layout = FRT_W_PLAIN;
      gq.N = L.nqkv; gq.K = H; gq.splits = L.s_qkv; gq.ksteps_per_split = H / kstep_of(d.dtype) / L.s_qkv;
      gq.a = a_qkv; gq.w = (const uint8_t*)c->wq[l]; gq.colscale = e4 ? c->sq[l] : nullptr;
      gq.act_scale = 1.f; gq.act_scale_ptr = actp(l, SITE_QKV); gq.partials = p_qkv; gq.epi = kEpiQkv;
      gq.q_out = qbuf; gq.k_out = kcl + (size_t)d.prefix_len * d.head_dim;
      gq.v_out = vcl + d.prefix_len; gq.v_ld = L.ldv; gq.nq = L.nattn; gq.hd = d.head_dim;

      GemmParams go = gq;
      go.N = H; go.K = L.nattn; go.splits = L.s_o; go.ksteps_per_split = L.nattn / kstep_of(d.dtype) / L.s_o;
      go.a = a_o; go.w = (const uint8_t*)c->wo[l]; go.colscale = e4 ? c->so[l] : nullptr;
      go.act_scale_ptr = actp(l, SITE_O); go.partials = p_o; go.epi = FRT_EPI_NONE; go.amax = nullptr;

      GemmParams gu = go;
      gu.N = 2 * F; gu.K = H; gu.splits = L.s_up; gu.ksteps_per_split = H / kstep_of(d.dtype) / L.s_up;
      gu.layout = FRT_W_GATE_UP; gu.a = a_up; gu.w = (const uint8_t*)c->wu[l]; gu.colscale = e4 ? c->su[l] : nullptr;
      gu.act_scale_ptr = actp(l, SITE_UP);
      gu.out_dtype = adt; gu.out_scale = 1.f; gu.out_scale_ptr = actp(l, SITE_DOWN);
      gu.amax = amax ? amax + l * 4 + SITE_DOWN : nullptr;
      if (L.s_up == 1) {
        gu.epi = FRT_EPI_SILU_GATE_QUANT; gu.out = a_down; gu.partials = nullptr;
      } else {
        gu.epi = FRT_EPI_NONE; gu.partials = (float*)at(c, L.p_up);
      }

      GemmParams gd = gu;
      gd.N = H; gd.K = F; gd.splits = L.s_down; gd.ksteps_per_split = F / kstep_of(d.dtype) / L.s_down;
      gd.layout = FRT_W_PLAIN; gd.a = a_down; gd.w = (const uint8_t*)c->wd[l]; gd.colscale = e4 ? c->sd[l] : nullptr;
      gd.act_scale_ptr = actp(l, SITE_DOWN); gd.epi = FRT_EPI_NONE; gd.partials = p_down; gd.out = nullptr;
      gd.amax = nullptr;

      // 1. producer: add the previous layer's MLP output, AdaRMSNorm (attention sublayer)
      RnqParams a{};
      a.M = M; a.K = H; a.MB = MB;
      a.x = pdown_prev; a.x_splits = pdown_prev ? L.s_down : 0;
      a.x_scale = 1.f; a.x_scale_ptr = pdown_prev ? actp(lp, SITE_DOWN) : nullptr;
      a.x_colscale = (pdown_prev && e4) ? c->sd[lp] : nullptr;
      a.residual = h_prev; a.residual_out = h_attn;
      a.gate = pdown_prev ? modp(kp, lp, 1, MOD_GATE) : nullptr;
      a.ada_scale = modp(k, l, 0, MOD_SCALE); a.ada_shift = modp(k, l, 0, MOD_SHIFT);
      a.eps = d.eps; a.out_dtype = adt; a.act_scale = 1.f; a.act_scale_ptr = actp(l, SITE_QKV);
      a.operand = a_qkv;
      a.amax = amax ? amax + l * 4 + SITE_QKV : nullptr;
      a.sink = sink;
      if (pf) {  // read the QKV GEMM's weights ahead
        a.touch = gemm_weight_touch(gq, 0, 1);
        a.touch_wgs = touch_wgs;
      }
      FRT_HIP(launch_rnq(a, s)); ++n;

      // 2. fused QKV GEMM: bf16 Q into its buffer, own K/V rows after the cached prefix
      FRT_HIP(launch_gemm(gq, s)); ++n;
      if (L.s_qkv > 1) {
        ReduceParams r{};
        r.M = M; r.N = L.nqkv; r.MB = MB; r.splits = L.s_qkv; r.partials = p_qkv;
        r.act_scale = 1.f; r.act_scale_ptr = actp(l, SITE_QKV); r.colscale = gq.colscale; r.epi = kEpiQkv;
        r.q_out = gq.q_out; r.k_out = gq.k_out; r.v_out = gq.v_out; r.nq = gq.nq; r.hd = gq.hd; r.v_ld = gq.v_ld;
        FRT_HIP(launch_reduce(r, s)); ++n;
      }

      if (dbg) {  // keep this step's own K/V rows for inspection
        const int nkv = M * d.head_dim;
        const size_t kvb = align256((size_t)nkv * 2);
        hipLaunchKernelGGL(copy_own_kv_kernel, dim3((nkv + 255) / 256), dim3(256), 0, s,
                           (const uint16_t*)gq.k_out, (const uint16_t*)gq.v_out, L.ldv, M, d.head_dim,
                           (uint16_t*)at(c, L.d_k, idx, kvb), (uint16_t*)at(c, L.d_v, idx, kvb));
        FRT_HIP(hipGetLastError()); ++n;
      }

      // 3. attention over [prefix ; own rows] -> O-projection operand
      AttnParams t{};
      t.M = M; t.MB = MB; t.n_heads = d.n_heads; t.kv_len = L.kv_len;
      t.q = qbuf; t.k = kcl; t.vt = vcl; t.ldv = L.ldv;
      t.out_dtype = adt; t.out_scale = 1.f; t.out_scale_ptr = actp(l, SITE_O);
      t.operand = a_o; t.workspace = (float*)at(c, L.aws);
      t.amax = amax ? amax + l * 4 + SITE_O : nullptr;
      if (L.fuse_o) {
        // 3+4. key chunks, then their merge fused with the O projection -> partials
        GemmParams gm = go;
        gm.ksteps = L.nattn / kstep_of(d.dtype);
        FRT_HIP(launch_attention_oproj(t, gm, s)); n += 2;
      } else {
        FRT_HIP(launch_attention(t, s)); n += attention_kernel_count(M, d.n_heads, L.kv_len);
        // 4. O projection -> partials
        FRT_HIP(launch_gemm(go, s)); ++n;
      }

      // 5. producer: gated residual of the attention output, AdaRMSNorm (MLP sublayer)
      RnqParams b = a;
      b.x = p_o; b.x_splits = L.s_o; b.x_scale_ptr = actp(l, SITE_O);
      b.x_colscale = e4 ? c->so[l] : nullptr;
      b.residual = h_attn; b.residual_out = h_mlp; b.gate = modp(k, l, 0, MOD_GATE);
      b.ada_scale = modp(k, l, 1, MOD_SCALE); b.ada_shift = modp(k, l, 1, MOD_SHIFT);
      b.act_scale_ptr = actp(l, SITE_UP); b.operand = a_up;
      b.amax = amax ? amax + l * 4 + SITE_UP : nullptr;
      if (pf) {
        b.touch = gemm_weight_touch(gd, 0, 1);
        b.touch_wgs = touch_wgs;
      }
      FRT_HIP(launch_rnq(b, s)); ++n;

      // 6. gate|up GEMM with SiLU(gate)*up + quantise (fused when not split)
      FRT_HIP(launch_gemm(gu, s)); ++n;
      if (L.s_up > 1) {
        ReduceParams r{};
        r.M = M; r.N = 2 * F; r.MB = MB; r.splits = L.s_up; r.partials = gu.partials;
        r.act_scale = 1.f; r.act_scale_ptr = actp(l, SITE_UP); r.colscale = gu.colscale;
        r.epi = FRT_EPI_SILU_GATE_QUANT; r.out = a_down; r.out_dtype = adt; r.out_scale = 1.f;
        r.out_scale_ptr = actp(l, SITE_DOWN); r.amax = gu.amax;
        FRT_HIP(launch_reduce(r, s)); ++n;
      }

      // 7. down projection -> partials, reduced by the next producer
      FRT_HIP(launch_gemm(gd, s)); ++n;

      h_prev = h_mlp;
      pdown_prev = p_down;
      kp = k;
      lp = l;
    }
  }
  // final gated residual of the last MLP output -> x_out
  RnqParams f{};
  f.M = M; f.K = H; f.MB = MB; f.x = pdown_prev; f.x_splits = L.s_down; f.x_scale = 1.f;
  f.x_scale_ptr = actp(lp, SITE_DOWN); f.x_colscale = e4 ? c->sd[lp] : nullptr;
  f.residual = h_prev; f.residual_out = (float*)at(c, L.x_out); f.gate = modp(kp, lp, 1, MOD_GATE);
  f.eps = d.eps; f.out_dtype = adt; f.act_scale = 1.f; f.operand = nullptr;
  FRT_HIP(launch_rnq(f, s)); ++n;
  if (count) *count = n;
  return FRT_OK;
}

extern "C" size_t frt_layer_chain_arena_bytes(const frt_chain_desc* desc) {
  if (validate_desc(desc) != FRT_OK) return 0;
  ChainLayout L;
  if (make_layout(desc, L) != FRT_OK) return 0;
  return L.total;
}

extern "C" int frt_layer_chain_create(const frt_chain_desc* desc, void* arena_dev, size_t arena_bytes,
                                      void* capture_stream, frt_chain** out) {
  FRT_CHECK(out, FRT_E_NULL);
  *out = nullptr;
  int st = validate_desc(desc);
  if (st) return st;
  FRT_CHECK(arena_dev, FRT_E_NULL);
  FRT_CHECK(aligned16(arena_dev), FRT_E_ALIGN);
  ChainLayout L;
  st = make_layout(desc, L);
  if (st) return st;
  FRT_CHECK(arena_bytes >= L.total, FRT_E_WORKSPACE);
  frt_chain* c = new (std::nothrow) frt_chain();
  FRT_CHECK(c, FRT_E_STATE);
  c->d = *desc;
  const int nl = desc->layers;
  c->wq.assign(desc->w_qkv, desc->w_qkv + nl);
  c->wo.assign(desc->w_o, desc->w_o + nl);
  c->wu.assign(desc->w_up, desc->w_up + nl);
  c->wd.assign(desc->w_down, desc->w_down + nl);
  if (desc->dtype == FRT_E4M3) {
    c->sq.assign(desc->s_qkv, desc->s_qkv + nl);
    c->so.assign(desc->s_o, desc->s_o + nl);
    c->su.assign(desc->s_up, desc->s_up + nl);
    c->sd.assign(desc->s_down, desc->s_down + nl);
  } else {
    c->sq.assign(nl, nullptr); c->so.assign(nl, nullptr); c->su.assign(nl, nullptr); c->sd.assign(nl, nullptr);
  }
  c->d.w_qkv = c->wq.data(); c->d.w_o = c->wo.data(); c->d.w_up = c->wu.data(); c->d.w_down = c->wd.data();
  c->d.s_qkv = c->sq.data(); c->d.s_o = c->so.data(); c->d.s_up = c->su.data(); c->d.s_down = c->sd.data();
  c->arena = (uint8_t*)arena_dev;
  c->arena_bytes = arena_bytes;
  c->L = L;
  c->kernels = 0;
  if (desc->use_graph) {
    hipStream_t cs = nullptr;
    hipError_t e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
    if (e != hipSuccess) { set_hip_error((int)e); delete c; return FRT_E_HIP; }
    if (capture_stream) {
      // order the capture after whatever the caller already queued
      hipEvent_t ev;
      if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) == hipSuccess) {
        (void)hipEventRecord(ev, (hipStream_t)capture_stream);
        (void)hipStreamWaitEvent(cs, ev, 0);
        (void)hipEventDestroy(ev);
      }
    }
    e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
    int n = 0;
    int rc = e == hipSuccess ? enqueue_chain(c, cs, &n) : FRT_E_HIP;
    hipGraph_t g = nullptr;
    hipError_t e2 = hipStreamEndCapture(cs, &g);
    if (e != hipSuccess) set_hip_error((int)e);
    if (rc == FRT_OK && e2 != hipSuccess) { set_hip_error((int)e2); rc = FRT_E_HIP; }
    if (rc == FRT_OK) {
      hipError_t e3 = hipGraphInstantiate(&c->exec, g, nullptr, nullptr, 0);
      if (e3 != hipSuccess) { set_hip_error((int)e3); rc = FRT_E_HIP; }
    }
    (void)hipStreamSynchronize(cs);
    (void)hipStreamDestroy(cs);
    if (rc != FRT_OK) {
      if (g) (void)hipGraphDestroy(g);
      delete c;
      return rc;
    }
    c->graph = g;
    c->kernels = n;
  } else {
    // count the launches without enqueueing anything
    const int attn_o = c->L.fuse_o ? 2 : attention_kernel_count(c->d.M, c->d.n_heads, c->L.kv_len) + 1;
    const int per_layer = 5 + attn_o + (c->L.s_up > 1) + (c->L.s_qkv > 1) + (c->d.keep_intermediates != 0);
    c->kernels = desc->steps * desc->layers * per_layer + 1;
  }
  *out = c;
  return FRT_OK;
}

extern "C" int frt_layer_chain_buffer(frt_chain* c, const char* name, void** dev, size_t* bytes) {
  FRT_CHECK(c && name, FRT_E_STATE);
  const ChainLayout& L = c->L;
  struct Named { const char* n; const Buf* b; } tab[] = {
      {"x_in", &L.x_in}, {"x_out", &L.x_out}, {"mod", &L.mod}, {"act_scale", &L.act},
      {"k_cache", &L.kc}, {"v_cache", &L.vc}, {"h", &L.h},
      {"dbg_h_attn", &L.d_h_attn}, {"dbg_h_mlp", &L.d_h_mlp}, {"dbg_a_qkv", &L.d_a_qkv},
      {"dbg_a_o", &L.d_a_o}, {"dbg_a_up", &L.d_a_up}, {"dbg_a_down", &L.d_a_down},
      {"dbg_p_o", &L.d_p_o}, {"dbg_p_down", &L.d_p_down}, {"dbg_q", &L.d_q},
      {"dbg_k_own", &L.d_k}, {"dbg_v_own", &L.d_v}};
  for (const Named& t : tab) {
    if (strcmp(t.n, name) == 0) {
      if (t.b->bytes == 0) return FRT_E_STATE;
      if (dev) *dev = c->arena + t.b->off;
      if (bytes) *bytes = t.b->bytes;
      return FRT_OK;
    }
  }
  return FRT_E_STATE;
}

extern "C" int frt_layer_chain_run(frt_chain* c, void* stream) {
  FRT_CHECK(c, FRT_E_STATE);
  hipStream_t s = (hipStream_t)stream;
  if (c->exec) {
    FRT_HIP(hipGraphLaunch(c->exec, s));
    return FRT_OK;
  }
  return enqueue_chain(c, s, nullptr);
}

extern "C" int frt_layer_chain_kernel_count(const frt_chain* c) { return c ? c->kernels : -1; }

// The persistent state is the arena's leading region, up to the first working buffer.
// A capsule holds that region followed by a 256-byte trailer whose first 16 bytes are a
// magic word and a token of the chain's shape fields and state layout, so a capsule is
// restored only into a chain whose state it fits.
constexpr size_t kTrailer = 256;
constexpr uint64_t kCapsuleMagic = 0x31555350'41435446ull;  // "FTCAPSU1" little-endian

static uint64_t layout_token(const frt_chain* c) {
  const frt_chain_desc& d = c->d;
  const ChainLayout& L = c->L;
  const uint64_t f[] = {(uint64_t)d.layers, (uint64_t)d.steps, (uint64_t)d.M, (uint64_t)d.hidden,
                        (uint64_t)d.n_heads, (uint64_t)d.head_dim, (uint64_t)d.prefix_len, (uint64_t)d.mlp,
                        (uint64_t)act_dtype_of(d.dtype), L.x_in.off, L.x_out.off, L.mod.off, L.act.off, L.kc.off,
                        L.vc.off, L.h.off};
  uint64_t h = 1469598103934665603ull;  // FNV-1a over the fields' bytes
  for (uint64_t v : f)
    for (int b = 0; b < 8; ++b) h = (h ^ ((v >> (8 * b)) & 0xffu)) * 1099511628211ull;
  return h;
}

__global__ void write_trailer_kernel(uint64_t* dst, uint64_t magic, uint64_t token) {
  if (threadIdx.x == 0) {
    dst[0] = magic;
    dst[1] = token;
  }
}

extern "C" size_t frt_layer_chain_state_bytes(const frt_chain* c) { return c ? c->L.h.off + kTrailer : 0; }

static int capsule_args(frt_chain* c, const void* capsule, size_t bytes) {
  FRT_CHECK(c, FRT_E_STATE);
  FRT_CHECK(capsule, FRT_E_NULL);
  FRT_CHECK(aligned16(capsule), FRT_E_ALIGN);
  FRT_CHECK(bytes == c->L.h.off + kTrailer, FRT_E_WORKSPACE);
  FRT_CHECK(!overlaps(capsule, bytes, c->arena, c->arena_bytes), FRT_E_ALIAS);
  return FRT_OK;
}

extern "C" int frt_layer_chain_snapshot(frt_chain* c, void* stream, void* capsule_dev, size_t capsule_bytes) {
  const int st = capsule_args(c, capsule_dev, capsule_bytes);
  if (st) return st;
  const size_t n = c->L.h.off;
  hipStream_t s = (hipStream_t)stream;
  FRT_HIP(hipMemcpyAsync(capsule_dev, c->arena, n, hipMemcpyDeviceToDevice, s));
  hipLaunchKernelGGL(write_trailer_kernel, dim3(1), dim3(64), 0, s, (uint64_t*)((uint8_t*)capsule_dev + n),
                     kCapsuleMagic, layout_token(c));
  FRT_HIP(hipGetLastError());
  return FRT_OK;
}

extern "C" int frt_layer_chain_restore(frt_chain* c, void* stream, const void* capsule_dev, size_t capsule_bytes) {
  const int st = capsule_args(c, capsule_dev, capsule_bytes);
  if (st) return st;
  const size_t n = c->L.h.off;
  hipStream_t s = (hipStream_t)stream;
  // the trailer is read back after whatever the stream already holds (the capsule may
  // have been written by work queued there), then checked on the host
  uint64_t trailer[2] = {0, 0};
  FRT_HIP(hipMemcpyAsync(trailer, (const uint8_t*)capsule_dev + n, sizeof trailer, hipMemcpyDeviceToHost, s));
  FRT_HIP(hipStreamSynchronize(s));
  FRT_CHECK(trailer[0] == kCapsuleMagic && trailer[1] == layout_token(c), FRT_E_STATE);
  FRT_HIP(hipMemcpyAsync(c->arena, capsule_dev, n, hipMemcpyDeviceToDevice, s));
  return FRT_OK;
}

__global__ void amax_to_scale_kernel(const unsigned* amax, float* scales, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) scales[i] = __builtin_bit_cast(float, amax[i]) / 448.0f;
}

extern "C" int frt_layer_chain_calibrate(frt_chain* c, void* stream, float* scales_dev) {
  FRT_CHECK(c, FRT_E_STATE);
  FRT_CHECK(c->d.dtype == FRT_BF16, FRT_E_DTYPE);
  FRT_CHECK(scales_dev, FRT_E_NULL);
  FRT_CHECK(aligned16(scales_dev), FRT_E_ALIGN);
  const int n = c->d.layers * 4;
  FRT_CHECK(!overlaps(scales_dev, (size_t)n * 4, c->arena, c->arena_bytes), FRT_E_ALIAS);
  hipStream_t s = (hipStream_t)stream;
  unsigned* amax = (unsigned*)at(c, c->L.amax);
  FRT_HIP(hipMemsetAsync(amax, 0, (size_t)n * 4, s));
  int rc = enqueue_chain(c, s, nullptr, amax);
  if (rc != FRT_OK) return rc;
  hipLaunchKernelGGL(amax_to_scale_kernel, dim3((n + 255) / 256), dim3(256), 0, s, (const unsigned*)amax, scales_dev, n);
  FRT_HIP(hipGetLastError());
  return FRT_OK;
}

extern "C" int frt_layer_chain_destroy(frt_chain* c) {
  FRT_CHECK(c, FRT_E_STATE);
  if (c->exec) (void)hipGraphExecDestroy(c->exec);
  if (c->graph) (void)hipGraphDestroy(c->graph);
  delete c;
  return FRT_OK;
}
