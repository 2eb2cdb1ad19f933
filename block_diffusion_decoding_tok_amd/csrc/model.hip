// Decoder context, forward, prefill and the block loop.
//
// Block loop (technical-report summary, "DiffusionGemma의 구성", flowchart;
// developer guide, "Block Autoregressive Diffusion"): canvas of random ids ->
// repeat {forward over the canvas with the canvas mask; LM head; sampler step}
// until every row is done -> one more forward of the final tokens writes every
// layer's K/V into cache slots [P, P + L) -> P += L.
//
// On a non-default stream the whole block (init, every step, commit) is
// captured once into a hipGraph per argument set and replayed; on the default
// stream it is launched eagerly.  Inside the graph nothing is allocated and no
// memset node is recorded (zeroing uses a fill kernel).
#include <map>
#include <tuple>
#include <vector>

#include "kernels.h"

namespace dg {

__global__ void fill_i32_kernel(int32_t* p, int n, int v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}
__global__ void copy_i32_kernel(const int32_t* s, int32_t* d, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) d[i] = s[i];
}

// Greedy token of each row: argmax over V logits (ties to the lowest id),
// written to tok[b] (the next step's input) and out[b * out_stride + col].
// One 1024-thread workgroup per row; each thread takes 8 values per 16-byte
// load, 8 loads in flight per batch (V % 8 == 0; bf16 or f32 logits).
// A NaN or infinite logit sets DG_STATUS_NONFINITE_LOGITS in *status.
template <typename T>
__global__ __launch_bounds__(1024) void argmax_rows_kernel(const T* __restrict__ logits, int V,
                                                           int32_t* __restrict__ tok,
                                                           int32_t* __restrict__ out,
                                                           int out_stride, int col,
                                                           int32_t* __restrict__ status) {
  constexpr int PER = 16 / sizeof(T);   // values per 16-byte load
  const int b = blockIdx.x, tid = threadIdx.x;
  const T* row = logits + static_cast<int64_t>(b) * V;
  const int npieces = V / PER;
  float best = -INFINITY;
  int bid = 0x7fffffff;
  bool finite = true;
  for (int p0 = tid; p0 < npieces; p0 += 1024 * 8) {
    uint4 u[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      u[j] = *reinterpret_cast<const uint4*>(row + static_cast<int64_t>(min(p0 + j * 1024, npieces - 1)) * PER);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int p = p0 + j * 1024;
      if (p >= npieces) continue;
      const T* e = reinterpret_cast<const T*>(&u[j]);
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        const float x = Elem<T>::load(e, q);
        const int v = p * PER + q;
        finite &= isfinite(x);
        const bool better = (x > best) | ((x == best) & (v < bid));
        best = better ? x : best;
        bid = better ? v : bid;
      }
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    const float ob = __shfl_xor(best, o);
    const int oi = __shfl_xor(bid, o);
    if (ob > best || (ob == best && oi < bid)) { best = ob; bid = oi; }
  }
  const bool nonfinite = __syncthreads_or(!finite);
  __shared__ float s_best[16];
  __shared__ int s_id[16];
  if ((tid & 63) == 0) { s_best[tid >> 6] = best; s_id[tid >> 6] = bid; }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 16; ++w)
      if (s_best[w] > best || (s_best[w] == best && s_id[w] < bid)) { best = s_best[w]; bid = s_id[w]; }
    if (bid == 0x7fffffff) bid = 0;     // every logit NaN: id 0
    tok[b] = bid;
    out[static_cast<int64_t>(b) * out_stride + col] = bid;
    if (nonfinite) atomicOr(status, DG_STATUS_NONFINITE_LOGITS);
  }
}

// Publishes the device status word of a block or AR run to the context's
// host-visible word (pinned host memory): a non-zero status is stored there,
// where the host finds it on a later call without synchronizing.
__global__ void publish_status_kernel(const int32_t* __restrict__ status,
                                      int32_t* __restrict__ host_word) {
  const int32_t v = *status;
  if (v) __hip_atomic_store(host_word, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

static dg_status fill_i32(int32_t* p, int n, int v, hipStream_t s) {
  fill_i32_kernel<<<(n + 255) / 256, 256, 0, s>>>(p, n, v);
  DG_LAUNCH_CHECK();
  return DG_OK;
}

}  // namespace dg

using namespace dg;

struct GraphKey {
  int B, Tmax, L, S, F;
  float t0, t1, eps, tc, tr;
  uint64_t seed;
  int policy;
  float bound;
  int part;                 // which piece of a block (adaptive mode: chunks of steps)
  std::vector<void*> ptrs;
  bool operator<(const GraphKey& o) const {
    return std::tie(B, Tmax, L, S, F, t0, t1, eps, tc, tr, seed, policy, bound, part, ptrs) <
           std::tie(o.B, o.Tmax, o.L, o.S, o.F, o.t0, o.t1, o.eps, o.tc, o.tr, o.seed, o.policy,
                    o.bound, o.part, o.ptrs);
  }
};

struct dg_ctx {
  dg_model_dims d;
  const void* emb = nullptr;
  const void* lm = nullptr;
  std::vector<const void*> wqkv, wo, wr, wgu, wd;
  std::vector<const float*> sgu, sd;
  int max_batch = 0, max_tokens = 0;
  int max_prefill = 0;             // tokens (all rows) per prefill forward
  // workspace carve-up
  float* x = nullptr;
  void* h = nullptr;
  void* qkv = nullptr;
  void* attn_out = nullptr;
  float* router = nullptr;
  int32_t* topk_ids = nullptr;
  float* gates = nullptr;
  int32_t* offsets = nullptr;
  int32_t* sorted_rows = nullptr;
  void* attn_ws = nullptr;
  void* moe_ws = nullptr;
  void* logits = nullptr;
  void* samp_ws = nullptr;
  int32_t* tokens = nullptr;
  uint8_t* committed = nullptr;
  uint8_t* renoised = nullptr;
  float* maxprob = nullptr;
  float* entropy = nullptr;
  float* mean_entropy = nullptr;
  int32_t* done = nullptr;
  int32_t* status = nullptr;
  int32_t* n_done = nullptr;       // rows of the current block that have stopped
  int32_t* active = nullptr;       // dg_generate: rows that have not met EOS
  int32_t* blk_tokens = nullptr;   // dg_generate: the current block's tokens [B, L]
  int32_t* blk_steps = nullptr;    // dg_generate: the current block's steps [B]
  float2* rope_tab = nullptr;      // (cos, sin) of a forward's tokens x pairs
  // deferred commit (dg_denoise_block_deferred): the last block's final
  // tokens, whose K/V the next deferred block's first step (or
  // dg_commit_pending) writes into the cache slots [P - L, P)
  int32_t* pending_tok = nullptr;  // [maxB, maxT]
  int32_t* fused_tok = nullptr;    // [maxB, 2 maxT]: each row's pending block, then its canvas
  int32_t* prefix_back = nullptr;  // [maxB]: prefix - L, the pending block's first position
  bool pending = false;            // host-side enqueue state
  int pending_B = 0, pending_L = 0, pending_Tmax = 0;
  std::vector<void*> pending_ptrs; // the caches and prefix array it belongs to
  // host-visible status word (pinned host memory): the device stores a
  // non-zero block status there; the host reads and clears it
  int32_t* host_status = nullptr;
  int32_t* host_status_dev = nullptr;    // its device-side address
  // host-visible copy of n_done, written at the end of each adaptive step
  int32_t* host_ndone = nullptr;
  int32_t* host_ndone_dev = nullptr;
  // the step gate of the steps being enqueued (adaptive mode only)
  StepGate gate;
  // graphs are captured on this private stream, never on the caller's
  hipStream_t cap_stream = nullptr;
  hipEvent_t step_ev[2] = {nullptr, nullptr};   // adaptive mode: steps in flight
  bool use_graphs = true;
  std::map<GraphKey, hipGraphExec_t> graphs;
  std::vector<const float*> router_override;   // empty: the model's own routing
  // the last MoE layer's gate-weighted slot rows still to be added into x
  // (host-side enqueue state: the next norm or the end of the forward does it)
  bool pending_combine = false;
  int router_override_tokens = 0;
};

namespace {

struct Layout {
  size_t x, h, qkv, attn_out, router, topk_ids, gates, offsets, sorted_rows, attn_ws, moe_ws,
      logits, samp_ws, tokens, committed, renoised, maxprob, entropy, mean_entropy, done, status,
      n_done, active, blk_tokens, blk_steps, rope_tab, pending_tok, fused_tok, prefix_back,
      total;
};

size_t esz(int dt) { return dt == DG_F32 ? 4 : 2; }

// The attention workspace of any forward the context runs: B <= maxB rows of
// n <= maxT tokens (canvas, AR, small prefill chunks) or of n <= maxP / B
// tokens (prefill chunks).
size_t attn_ws_max(const dg_model_dims& d, int maxB, int maxT, int maxP) {
  size_t m = 0;
  for (int B = 1; B <= maxB; ++B)
    for (int n = 1; n <= std::max(maxT, maxP / B); ++n)
      m = std::max(m, attention_workspace_bytes(B, n, d.n_heads, d.n_kv_heads, d.head_dim,
                                                1 << 30, d.act_dtype));
  return m;
}

// maxP: tokens (all rows) of one prefill forward; the activation buffers
// hold max(maxB * maxT, maxP) tokens, the canvas state and logits maxB * maxT.
Layout layout(const dg_model_dims& d, int maxB, int maxT, int maxP) {
  Layout L{};
  const size_t Tc = static_cast<size_t>(maxB) * maxT;
  const size_t T = std::max(Tc, static_cast<size_t>(maxP));
  const size_t qkv_w = static_cast<size_t>(d.n_heads + 2 * d.n_kv_heads) * d.head_dim;
  const size_t a = esz(d.act_dtype);
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += align_up(bytes, 256); return o; };
  const size_t T16 = align_up(T, 16);     // the tiled activation layout's whole token blocks
  L.x = take(T * d.d_model * 4);
  L.h = take(T16 * d.d_model * a);
  L.qkv = take(T * qkv_w * a);
  L.attn_out = take(T16 * d.n_heads * d.head_dim * a);
  L.router = take(T * d.n_experts * 4);
  L.topk_ids = take(T * d.top_k * 4);
  L.gates = take(T * d.top_k * 4);
  L.offsets = take((d.n_experts + 1) * 4);
  L.sorted_rows = take(T * d.top_k * 4);
  L.attn_ws = take(attn_ws_max(d, maxB, maxT, maxP));
  L.moe_ws = take(std::max(moe_ffn_workspace_bytes(static_cast<int>(T), d.d_model, d.d_ff,
                                                   d.n_experts, d.top_k, d.act_dtype),
                           moe_route_workspace_bytes(static_cast<int>(T), d.n_experts, d.top_k)));
  L.logits = take(Tc * d.vocab * a);
  L.samp_ws = take(sampler_workspace_bytes(maxB, maxT, d.vocab));
  L.tokens = take(T * 4);            // also stages a prefill chunk's ids
  L.committed = take(Tc);
  L.renoised = take(Tc);
  L.maxprob = take(Tc * 4);
  L.entropy = take(Tc * 4);
  L.mean_entropy = take(maxB * 4);
  L.done = take(maxB * 4);
  L.status = take(4);
  L.n_done = take(4);
  L.active = take(maxB * 4);
  L.blk_tokens = take(Tc * 4);
  L.blk_steps = take(maxB * 4);
  L.rope_tab = take(T * (d.head_dim / 2) * sizeof(float2));   // RoPE table of a forward
  L.pending_tok = take(Tc * 4);
  L.fused_tok = take(2 * Tc * 4);
  L.prefix_back = take(maxB * 4);
  L.total = off;
  return L;
}

dg_status check_dims(const dg_model_dims* d) {
  DG_CHECK_ARG(d != nullptr, "dims is null");
  DG_CHECK_SHAPE(d->n_layers > 0 && d->d_model > 0 && d->n_heads > 0 && d->n_kv_heads > 0 &&
                     d->head_dim > 0 && d->n_experts > 0 && d->top_k > 0 && d->d_ff > 0 &&
                     d->vocab > 0,
                 "dims must be positive");
  DG_CHECK_SHAPE(d->n_heads % d->n_kv_heads == 0, "n_heads must be a multiple of n_kv_heads");
  DG_CHECK_SHAPE(d->n_experts <= 256 && d->top_k <= d->n_experts && d->top_k <= 16,
                 "need n_experts <= 256 and top_k <= min(n_experts, 16)");
  DG_CHECK_SHAPE(d->vocab % 8 == 0, "vocab must be a multiple of 8");
  DG_CHECK_ARG(d->rope_theta > 1.f, "rope_theta must be > 1");
  DG_CHECK_ARG(d->weight_layout == DG_LAYOUT_ROWMAJOR ||
                   (d->weight_layout == DG_LAYOUT_TILED && d->act_dtype == DG_BF16),
               "weight_layout must be row-major, or tiled with bf16 activations");
  if (d->act_dtype == DG_BF16) {
    DG_CHECK_ARG(d->expert_dtype == DG_BF16 || d->expert_dtype == DG_FP8_E4M3 ||
                     (d->expert_dtype == DG_MXFP4 && d->weight_layout == DG_LAYOUT_TILED),
                 "bf16 activations need bf16, fp8 or (tiled) MXFP4 experts");
    DG_CHECK_SHAPE(d->head_dim == 128, "the bf16 path needs head_dim 128");
    const int qkv_n = (d->n_heads + 2 * d->n_kv_heads) * d->head_dim;
    DG_CHECK_SHAPE(d->d_model % 128 == 0 && qkv_n % 128 == 0 && d->n_experts % 128 == 0 &&
                       d->vocab % 128 == 0 && (d->n_heads * d->head_dim) % 64 == 0 &&
                       d->d_ff % 64 == 0,
                   "the bf16 path needs d_model, QKV width, n_experts, vocab % 128 == 0 "
                   "and attention width, d_ff % 64 == 0");
  } else {
    DG_CHECK_ARG(d->act_dtype == DG_F32 && d->expert_dtype == DG_F32,
                 "act_dtype must be DG_BF16 or DG_F32 (f32 needs f32 experts)");
    DG_CHECK_SHAPE(d->head_dim % 2 == 0 && d->head_dim <= 128, "f32 head_dim must be even, <= 128");
    DG_CHECK_SHAPE(d->d_model % 4 == 0, "d_model must be a multiple of 4");
  }
  return DG_OK;
}

dg_status norm_input(dg_ctx* c, int T, hipStream_t s, bool tiled = false,
                     const RopeTable& rope = {}, const NormRows& rows = {}, int m_out = 0);
dg_status layer_tail(dg_ctx* c, int l, int B, int n, bool xt, hipStream_t s);

// Whether a layer over T tokens runs its dense projections on the tiled
// activation layout: the fused QKV + RoPE projection and the O projection
// both take it (bf16, tiled weights, heads of 128, more than 16 tokens).
bool tiled_acts(const dg_model_dims& d, const QkvRope& r) {
  const int qd = d.n_heads * d.head_dim;
  return d.act_dtype == DG_BF16 && d.weight_layout == DG_LAYOUT_TILED && d.d_model % 64 == 0 &&
         d.d_model / 4 <= 1024 && qkv_rope_supported(r, d.d_model) &&
         dense_xt_supported(r.B * r.Lq, d.d_model, qd);
}

// One decoder layer over T = B * n tokens (residual ctx->x).
dg_status layer(dg_ctx* c, int l, int B, int n, void* kc, void* vc, int Tmax,
                const int32_t* prefix_len, int mode, bool kv_only, hipStream_t s,
                int mask_blk = 0) {
  const dg_model_dims& d = c->d;
  const int T = B * n;
  const int qd = d.n_heads * d.head_dim, kd = d.n_kv_heads * d.head_dim;
  const int qkv_w = qd + 2 * kd;
  const size_t a = esz(d.act_dtype);
  dg_status st;
  QkvRope r{prefix_len, B, n, d.n_heads, d.n_kv_heads, d.head_dim, Tmax, d.rope_theta,
            c->attn_ws, kc, vc, 0, c->rope_tab};
  const bool xt = tiled_acts(d, r);
  r.x_tiled = xt ? 1 : 0;
  // the input norm also writes the RoPE angles the fused QKV projection reads
  RopeTable rt;
  if (d.act_dtype == DG_BF16 && qkv_rope_supported(r, d.d_model))
    rt = RopeTable{prefix_len, n, d.head_dim / 2, d.rope_theta, c->rope_tab};
  if ((st = norm_input(c, T, s, xt, rt))) return st;
  // bf16: the projection rotates q and k in its epilogue and writes q to the
  // attention workspace, k and v to the caches (one launch less per layer)
  if (d.act_dtype == DG_BF16) {
    st = launch_qkv_rope(c->h, c->wqkv[l], d.d_model, d.weight_layout, r, s, c->gate);
    if (st == DG_OK) {
      if (kv_only) return DG_OK;
      AttnArgs aa{nullptr, nullptr, nullptr, 0, 0, kc, vc, prefix_len, B, n, d.n_heads,
                  d.n_kv_heads, d.head_dim, Tmax, mode, d.rope_theta, d.act_dtype, c->attn_out, 1,
                  xt ? 1 : 0, c->gate, mask_blk};
      if ((st = launch_attention(aa, c->attn_ws, s))) return st;
      return layer_tail(c, l, B, n, xt, s);
    }
    if (st != DG_ERR_UNSUPPORTED || xt) return st;
  }
  if ((st = launch_gemm(c->h, c->wqkv[l], c->qkv, T, qkv_w, d.d_model, d.act_dtype,
                        d.weight_layout, d.act_dtype, kStore, s)))
    return st;
  char* qkv = static_cast<char*>(c->qkv);
  if (kv_only)
    return launch_commit(qkv + qd * a, qkv + (qd + kd) * a, qkv_w, kc, vc,
                         const_cast<int32_t*>(prefix_len), B, n, d.n_kv_heads, d.head_dim, Tmax,
                         d.rope_theta, d.act_dtype, false, s);
  AttnArgs aa{qkv, qkv + qd * a, qkv + (qd + kd) * a, qkv_w, qkv_w, kc, vc, prefix_len, B, n,
              d.n_heads, d.n_kv_heads, d.head_dim, Tmax, mode, d.rope_theta, d.act_dtype,
              c->attn_out, 0, 0, c->gate, mask_blk};
  if ((st = launch_attention(aa, c->attn_ws, s))) return st;
  return layer_tail(c, l, B, n, false, s);
}

// The rest of a layer after attention: O projection + residual, RMSNorm,
// router, routing, expert gate/up and down (the combine waits for the next
// norm).  xt: the attention output is in the tiled activation layout.
dg_status layer_tail(dg_ctx* c, int l, int B, int n, bool xt, hipStream_t s) {
  const dg_model_dims& d = c->d;
  const int T = B * n;
  const int qd = d.n_heads * d.head_dim;
  dg_status st;
  if (xt) {
    if ((st = launch_gemm_xt(c->attn_out, c->wo[l], c->x, T, d.d_model, qd, DG_F32,
                             kAccumulateF32, s, c->gate)))
      return st;
  } else if ((st = launch_gemm(c->attn_out, c->wo[l], c->x, T, d.d_model, qd, d.act_dtype,
                               d.weight_layout, DG_F32, kAccumulateF32, s, c->gate))) {
    return st;
  }
  if ((st = launch_rmsnorm(c->x, c->h, T, d.d_model, d.act_dtype, s))) return st;
  if ((st = launch_gemm(c->h, c->wr[l], c->router, T, d.n_experts, d.d_model, d.act_dtype,
                        d.weight_layout, DG_F32, kStore, s, c->gate)))
    return st;
  const float* route_in = c->router_override.empty() ? c->router : c->router_override[l];
  if ((st = launch_moe_route(route_in, T, d.n_experts, d.top_k, c->topk_ids, c->gates,
                             c->offsets, c->sorted_rows, c->moe_ws, s)))
    return st;
  // gate/up and down now; the combine into x is left to the next norm
  void *h_mid, *y_slot;
  moe_ffn_workspace_split(c->moe_ws, T, d.d_ff, d.top_k, d.act_dtype, &h_mid, &y_slot);
  if ((st = launch_moe_gate_up(c->h, d.act_dtype, c->wgu[l], d.expert_dtype, d.weight_layout,
                               c->sgu[l], c->offsets, c->sorted_rows, T, d.d_model, d.d_ff,
                               d.n_experts, d.top_k, h_mid, s, c->gate)))
    return st;
  if ((st = launch_moe_down(h_mid, d.act_dtype, c->wd[l], d.expert_dtype, d.weight_layout,
                            c->sd[l], c->gates, c->offsets, c->sorted_rows, T, d.d_model, d.d_ff,
                            d.n_experts, d.top_k, y_slot, s, c->gate)))
    return st;
  c->pending_combine = true;
  return DG_OK;
}

// RMSNorm of the residual stream into c->h (tiled: in the tiled activation
// layout), taking a pending MoE combine (the previous layer's expert outputs)
// into x first.
// The norm of a forward's T tokens into c->h (m_out rows through `rows` when
// set), with the last MoE layer's pending combine.
dg_status norm_input(dg_ctx* c, int T, hipStream_t s, bool tiled, const RopeTable& rope,
                     const NormRows& rows, int m_out) {
  const dg_model_dims& d = c->d;
  void *h_mid, *y_slot = nullptr;
  if (c->pending_combine)
    moe_ffn_workspace_split(c->moe_ws, T, d.d_ff, d.top_k, d.act_dtype, &h_mid, &y_slot);
  c->pending_combine = false;
  return launch_combine_rmsnorm(y_slot, d.act_dtype, d.top_k, c->x, c->h,
                                m_out > 0 ? m_out : T, d.d_model, d.act_dtype, s, tiled, rope,
                                rows);
}

// Flush a pending MoE combine into x (end of a forward without the LM head).
dg_status flush_combine(dg_ctx* c, int T, hipStream_t s) {
  if (!c->pending_combine) return DG_OK;
  const dg_model_dims& d = c->d;
  void *h_mid, *y_slot;
  moe_ffn_workspace_split(c->moe_ws, T, d.d_ff, d.top_k, d.act_dtype, &h_mid, &y_slot);
  c->pending_combine = false;
  return launch_moe_combine(y_slot, d.act_dtype, T, d.d_model, d.top_k, c->x, s);
}

// mask_blk > 0: block-causal attention over the n tokens of each row in
// groups of mask_blk; lm_rows: the rows of each batch row the LM head takes
// (logits [B * lm_rows.blk] when set, else all B * n).
dg_status forward(dg_ctx* c, const int32_t* tokens, int B, int n, int l0, int l1,
                  void* const* kcs, void* const* vcs, int Tmax, const int32_t* prefix_len,
                  int mode, void* logits, bool commit_only, hipStream_t s, int mask_blk = 0,
                  const NormRows& lm_rows = {}) {
  const dg_model_dims& d = c->d;
  dg_status st;
  c->pending_combine = false;   // a combine is only carried within one forward
  if (tokens && (st = launch_embed(tokens, c->emb, c->x, B * n, d.d_model, d.act_dtype, s)))
    return st;
  for (int l = l0; l < l1; ++l) {
    const bool kv_only = commit_only && l == d.n_layers - 1;
    if ((st = layer(c, l, B, n, kcs[l], vcs[l], Tmax, prefix_len, mode, kv_only, s, mask_blk)))
      return st;
  }
  if (!logits) return flush_combine(c, B * n, s);
  const int m = lm_rows.blk > 0 ? B * lm_rows.blk : B * n;
  if ((st = norm_input(c, B * n, s, false, {}, lm_rows, m))) return st;
  return launch_gemm(c->h, c->lm, logits, m, d.vocab, d.d_model, d.act_dtype, d.weight_layout,
                     d.act_dtype, kStore, s, c->gate);
}

// Copies the count of stopped rows to the context's host-visible word.
__global__ void publish_count_kernel(const int32_t* __restrict__ n_done,
                                     int32_t* __restrict__ host_word) {
  __hip_atomic_store(host_word, *n_done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

dg_status publish_status(dg_ctx* c, hipStream_t s) {
  publish_status_kernel<<<1, 1, 0, s>>>(c->status, c->host_status_dev);
  DG_LAUNCH_CHECK();
  return DG_OK;
}

// A block in three pieces: begin (canvas init), steps [s0, s1) (forward +
// LM head + sampler each), end (commit forward, prefix advance, tokens out).
dg_status enqueue_block_begin(dg_ctx* c, const dg_sampler_cfg& cfg, int B,
                              const int32_t* prefix_len, int32_t* steps_taken, hipStream_t s) {
  dg_status st;
  if ((st = launch_init_canvas(prefix_len, B, cfg.canvas_len, c->d.vocab, cfg.seed, c->tokens,
                               c->committed, c->done, s)))
    return st;
  if ((st = fill_i32(steps_taken, B, 0, s))) return st;
  if ((st = fill_i32(c->n_done, 1, 0, s))) return st;
  return fill_i32(c->status, 1, 0, s);
}

dg_status enqueue_block_steps(dg_ctx* c, const dg_sampler_cfg& cfg, int B, void* const* kcs,
                              void* const* vcs, int Tmax, int32_t* prefix_len,
                              int32_t* steps_taken, int s0, int s1, hipStream_t s) {
  const dg_model_dims& d = c->d;
  const int L = cfg.canvas_len;
  dg_status st;
  for (int step = s0; step < s1; ++step) {
    if ((st = forward(c, c->tokens, B, L, 0, d.n_layers, kcs, vcs, Tmax, prefix_len,
                      DG_MASK_CANVAS, c->logits, false, s)))
      return st;
    if ((st = launch_sampler(c->logits, d.act_dtype, B, L, d.vocab, step, cfg, prefix_len,
                             c->tokens, c->committed, c->renoised, c->maxprob, c->entropy,
                             c->mean_entropy, c->done, c->status, steps_taken, c->samp_ws, s,
                             c->n_done)))
      return st;
  }
  return DG_OK;
}

dg_status enqueue_block_end(dg_ctx* c, const dg_sampler_cfg& cfg, int B, void* const* kcs,
                            void* const* vcs, int Tmax, int32_t* prefix_len, int32_t* tokens_out,
                            hipStream_t s) {
  const int L = cfg.canvas_len;
  dg_status st;
  // commit: the final tokens' K/V of every layer into slots [P, P + L)
  if ((st = forward(c, c->tokens, B, L, 0, c->d.n_layers, kcs, vcs, Tmax, prefix_len,
                    DG_MASK_CANVAS, nullptr, true, s)))
    return st;
  if ((st = launch_advance_prefix(prefix_len, B, L, s))) return st;
  copy_i32_kernel<<<(B * L + 255) / 256, 256, 0, s>>>(c->tokens, tokens_out, B * L);
  DG_LAUNCH_CHECK();
  return publish_status(c, s);
}

// Deferred commit: row b's pending block then its canvas, [B, 2L]; and the
// pending block's first position, prefix - L.
__global__ void assemble_fused_kernel(const int32_t* __restrict__ pending,
                                      const int32_t* __restrict__ canvas, int B, int L,
                                      int32_t* __restrict__ fused) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * 2 * L) return;
  const int b = i / (2 * L), j = i % (2 * L);
  fused[i] = j < L ? pending[b * L + j] : canvas[b * L + j - L];
}

__global__ void prefix_back_kernel(const int32_t* __restrict__ prefix_len, int B, int L,
                                   int32_t* __restrict__ back) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) back[b] = prefix_len[b] - L;
}

// The first step of a deferred block with a commit pending: one forward over
// each row's pending block (positions [P - L, P)) followed by its canvas
// ([P, P + L)), the pending block attending to the cache before it and to
// itself, the canvas to both blocks and itself (block-causal groups of L).
// It writes the pending block's K/V into the cache as its commit forward
// would, and the canvas rows' logits as the step's own forward would; then
// the step's sampler.
dg_status enqueue_fused_first_step(dg_ctx* c, const dg_sampler_cfg& cfg, int B, void* const* kcs,
                                   void* const* vcs, int Tmax, int32_t* prefix_len,
                                   int32_t* steps_taken, hipStream_t s) {
  const dg_model_dims& d = c->d;
  const int L = cfg.canvas_len;
  assemble_fused_kernel<<<(2 * B * L + 255) / 256, 256, 0, s>>>(c->pending_tok, c->tokens, B, L,
                                                                c->fused_tok);
  DG_LAUNCH_CHECK();
  prefix_back_kernel<<<(B + 63) / 64, 64, 0, s>>>(prefix_len, B, L, c->prefix_back);
  DG_LAUNCH_CHECK();
  dg_status st;
  if ((st = forward(c, c->fused_tok, B, 2 * L, 0, d.n_layers, kcs, vcs, Tmax, c->prefix_back,
                    DG_MASK_CANVAS, c->logits, false, s, L, NormRows{L, 2 * L, L})))
    return st;
  return launch_sampler(c->logits, d.act_dtype, B, L, d.vocab, 0, cfg, prefix_len, c->tokens,
                        c->committed, c->renoised, c->maxprob, c->entropy, c->mean_entropy,
                        c->done, c->status, steps_taken, c->samp_ws, s, c->n_done);
}

// The commit forward of the pending block alone (positions [P - L, P)).
dg_status enqueue_commit_pending(dg_ctx* c, int B, int L, void* const* kcs, void* const* vcs,
                                 int Tmax, const int32_t* prefix_len, hipStream_t s) {
  prefix_back_kernel<<<(B + 63) / 64, 64, 0, s>>>(prefix_len, B, L, c->prefix_back);
  DG_LAUNCH_CHECK();
  return forward(c, c->pending_tok, B, L, 0, c->d.n_layers, kcs, vcs, Tmax, c->prefix_back,
                 DG_MASK_CANVAS, nullptr, true, s);
}

// A fixed-steps block whose commit is deferred: its first step fused with
// the previous block's commit when one is pending; at the end the final
// tokens become the pending block and the prefix advances by L.
dg_status enqueue_block_deferred(dg_ctx* c, const dg_sampler_cfg& cfg, int B, void* const* kcs,
                                 void* const* vcs, int Tmax, int32_t* prefix_len,
                                 int32_t* tokens_out, int32_t* steps_taken, bool fused,
                                 hipStream_t s) {
  const int L = cfg.canvas_len;
  const int n_steps = cfg.fixed_steps;
  dg_status st;
  if ((st = enqueue_block_begin(c, cfg, B, prefix_len, steps_taken, s))) return st;
  int first = 0;
  if (fused) {
    if ((st = enqueue_fused_first_step(c, cfg, B, kcs, vcs, Tmax, prefix_len, steps_taken, s)))
      return st;
    first = 1;
  }
  if ((st = enqueue_block_steps(c, cfg, B, kcs, vcs, Tmax, prefix_len, steps_taken, first,
                                n_steps, s)))
    return st;
  copy_i32_kernel<<<(B * L + 255) / 256, 256, 0, s>>>(c->tokens, c->pending_tok, B * L);
  DG_LAUNCH_CHECK();
  if ((st = launch_advance_prefix(prefix_len, B, L, s))) return st;
  copy_i32_kernel<<<(B * L + 255) / 256, 256, 0, s>>>(c->tokens, tokens_out, B * L);
  DG_LAUNCH_CHECK();
  return publish_status(c, s);
}

dg_status enqueue_block(dg_ctx* c, const dg_sampler_cfg& cfg, int B, void* const* kcs,
                        void* const* vcs, int Tmax, int32_t* prefix_len, int32_t* tokens_out,
                        int32_t* steps_taken, hipStream_t s) {
  const int n_steps = cfg.fixed_steps > 0 ? cfg.fixed_steps : cfg.max_steps;
  dg_status st;
  if ((st = enqueue_block_begin(c, cfg, B, prefix_len, steps_taken, s))) return st;
  if ((st = enqueue_block_steps(c, cfg, B, kcs, vcs, Tmax, prefix_len, steps_taken, 0, n_steps, s)))
    return st;
  return enqueue_block_end(c, cfg, B, kcs, vcs, Tmax, prefix_len, tokens_out, s);
}

// R29: n_steps greedy single-token causal steps; c->tokens holds each row's
// current input token.
dg_status enqueue_ar(dg_ctx* c, int B, int n_steps, const int32_t* tokens_in, void* const* kcs,
                     void* const* vcs, int Tmax, int32_t* prefix_len, int32_t* tokens_out,
                     hipStream_t s) {
  const dg_model_dims& d = c->d;
  copy_i32_kernel<<<(B + 255) / 256, 256, 0, s>>>(tokens_in, c->tokens, B);
  DG_LAUNCH_CHECK();
  dg_status st;
  if ((st = fill_i32(c->status, 1, 0, s))) return st;
  for (int step = 0; step < n_steps; ++step) {
    if ((st = forward(c, c->tokens, B, 1, 0, d.n_layers, kcs, vcs, Tmax, prefix_len,
                      DG_MASK_CAUSAL, c->logits, false, s)))
      return st;
    if (d.act_dtype == DG_BF16)
      argmax_rows_kernel<bf16_t><<<B, 1024, 0, s>>>(static_cast<const bf16_t*>(c->logits),
                                                    d.vocab, c->tokens, tokens_out, n_steps, step,
                                                    c->status);
    else
      argmax_rows_kernel<float><<<B, 1024, 0, s>>>(static_cast<const float*>(c->logits), d.vocab,
                                                   c->tokens, tokens_out, n_steps, step,
                                                   c->status);
    DG_LAUNCH_CHECK();
    if ((st = launch_advance_prefix(prefix_len, B, 1, s))) return st;
  }
  return publish_status(c, s);
}

// Reports (and clears) a non-finite status the device stored in the
// context's host word: DG_ERR_NONFINITE, else DG_OK.  No synchronization.
dg_status take_status(dg_ctx* c, const char* fn) {
  const int32_t v = __atomic_exchange_n(c->host_status, 0, __ATOMIC_ACQ_REL);
  if (v & DG_STATUS_NONFINITE_LOGITS)
    return fail(DG_ERR_NONFINITE, std::string(fn) +
                                      ": non-finite logits (NaN or Inf) in a block or AR run "
                                      "queued earlier on this context");
  return DG_OK;
}

dg_status check_run(dg_ctx* c, int B, int n, void* const* kcs, void* const* vcs, int Tmax,
                    const int32_t* prefix_len, const char* fn, int max_n = 0) {
  if (max_n == 0 && c) max_n = c->max_tokens;
  DG_CHECK_ARG(c != nullptr, std::string(fn) + ": ctx is null");
  DG_CHECK_ARG(kcs && vcs && prefix_len, std::string(fn) + ": null pointer");
  for (int l = 0; l < c->d.n_layers; ++l)
    DG_CHECK_ARG(kcs[l] && vcs[l], std::string(fn) + ": null cache pointer");
  DG_CHECK_SHAPE(B > 0 && B <= c->max_batch, std::string(fn) + ": B outside [1, max_batch]");
  DG_CHECK_SHAPE(n > 0 && n <= max_n, std::string(fn) + ": n outside [1, max_tokens]");
  DG_CHECK_SHAPE(Tmax >= n, std::string(fn) + ": Tmax smaller than the block");
  DG_CHECK_SHAPE(c->router_override.empty() || B * n <= c->router_override_tokens,
                 std::string(fn) + ": more tokens than the router override holds");
  return DG_OK;
}

// Launch what enq(stream) enqueues: captured once per key into a hipGraph
// (on the context's private capture stream, so the caller's stream and the
// work already queued on it are never part of a capture) and replayed on s
// when graphs are on and s is not the null stream, else enqueued directly.
template <typename F>
dg_status run_graph(dg_ctx* ctx, const GraphKey& key, hipStream_t s, F&& enq) {
  if (!ctx->use_graphs || s == nullptr) return enq(s);
  auto it = ctx->graphs.find(key);
  if (it == ctx->graphs.end()) {
    hipStream_t cs = ctx->cap_stream;
    DG_HIP(hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal));
    const dg_status st = enq(cs);
    hipGraph_t g = nullptr;
    hipError_t e = hipStreamEndCapture(cs, &g);
    if (st != DG_OK) {
      if (g) (void)hipGraphDestroy(g);
      return st;
    }
    if (e != hipSuccess)
      return fail(DG_ERR_HIP, std::string("hipStreamEndCapture: ") + hipGetErrorString(e));
    hipGraphExec_t exec = nullptr;
    e = hipGraphInstantiate(&exec, g, nullptr, nullptr, 0);
    (void)hipGraphDestroy(g);
    if (e != hipSuccess)
      return fail(DG_ERR_HIP, std::string("hipGraphInstantiate: ") + hipGetErrorString(e));
    it = ctx->graphs.emplace(key, exec).first;
  }
  DG_HIP(hipGraphLaunch(it->second, s));
  return DG_OK;
}

dg_status check_block_cfg(const dg_sampler_cfg* cfg, const char* fn) {
  DG_CHECK_SHAPE(cfg->max_steps >= 1 && cfg->fixed_steps >= 0 && cfg->fixed_steps <= cfg->max_steps,
                 std::string(fn) + ": bad step settings");
  DG_CHECK_ARG(cfg->temp_start > 0.f && cfg->temp_end > 0.f, std::string(fn) + ": bad temperatures");
  DG_CHECK_ARG(cfg->commit_policy == DG_COMMIT_MAXPROB ||
                   (cfg->commit_policy == DG_COMMIT_ENTROPY_BOUND && cfg->entropy_bound >= 0.f &&
                    cfg->entropy_bound < INFINITY),
               std::string(fn) + ": bad commit_policy / entropy_bound");
  return DG_OK;
}

// Every entry point but the deferred block and dg_commit_pending refuses to
// run while a deferred commit is pending (its K/V are not in the cache yet).
dg_status check_no_pending(dg_ctx* c, const char* fn) {
  if (c && c->pending)
    return fail(DG_ERR_INVALID_ARG, std::string(fn) +
                                        ": a deferred block commit is pending on this context "
                                        "(call dg_commit_pending first)");
  return DG_OK;
}

// The caches, prefix array, B, L and Tmax a pending commit belongs to.
std::vector<void*> pending_key_ptrs(dg_ctx* c, void* const* kcs, void* const* vcs,
                                    const int32_t* prefix_len) {
  std::vector<void*> v;
  for (int l = 0; l < c->d.n_layers; ++l) {
    v.push_back(kcs[l]);
    v.push_back(vcs[l]);
  }
  v.push_back(const_cast<int32_t*>(prefix_len));
  return v;
}

// Adaptive mode: steps the host keeps queued beyond the one whose done
// count it waits for.  The device gates every heavy kernel of a queued step
// on that count, so a step queued after the block ended costs only its
// launches.
constexpr int kAdaptiveLookahead = 1;

// One block (see dg_denoise_block).  part keys: 0 the whole fixed-steps
// block; 1 + s the adaptive step s (with the canvas init when s == 0); -2
// the commit.
dg_status run_block(dg_ctx* c, const dg_sampler_cfg& cfg, int B, void* const* kcs,
                    void* const* vcs, int Tmax, int32_t* prefix_len, int32_t* tokens_out,
                    int32_t* steps_taken, hipStream_t s) {
  GraphKey key{B, Tmax, cfg.canvas_len, cfg.max_steps, cfg.fixed_steps, cfg.temp_start,
               cfg.temp_end, cfg.stop_entropy, cfg.commit_prob, cfg.renoise_prob, cfg.seed,
               cfg.commit_policy, cfg.entropy_bound, 0, {}};
  for (int l = 0; l < c->d.n_layers; ++l) {
    key.ptrs.push_back(kcs[l]);
    key.ptrs.push_back(vcs[l]);
  }
  key.ptrs.push_back(prefix_len);
  key.ptrs.push_back(tokens_out);
  key.ptrs.push_back(steps_taken);
  if (cfg.fixed_steps > 0)
    return run_graph(c, key, s, [&](hipStream_t q) {
      return enqueue_block(c, cfg, B, kcs, vcs, Tmax, prefix_len, tokens_out, steps_taken, q);
    });
  // Adaptive: one graph per step, each gated on the device by the count of
  // stopped rows (and attention per row by the row's done flag) and ending
  // with that count copied to a host-visible word.  The host keeps
  // kAdaptiveLookahead steps queued beyond the one it waits for (an event
  // after each step), so the device never idles on the host's check; the
  // steps queued past the block's end run gated.
  const int S = cfg.max_steps;
  dg_status st;
  auto launch_step = [&](int step) -> dg_status {
    key.part = 1 + step;
    dg_status r = run_graph(c, key, s, [&](hipStream_t q) {
      dg_status e = DG_OK;
      if (step == 0 && (e = enqueue_block_begin(c, cfg, B, prefix_len, steps_taken, q))) return e;
      c->gate = StepGate{c->n_done, B, c->done};
      e = enqueue_block_steps(c, cfg, B, kcs, vcs, Tmax, prefix_len, steps_taken, step, step + 1,
                              q);
      c->gate = StepGate{};
      if (e != DG_OK) return e;
      if ((e = publish_status(c, q))) return e;
      publish_count_kernel<<<1, 1, 0, q>>>(c->n_done, c->host_ndone_dev);
      DG_LAUNCH_CHECK();
      return DG_OK;
    });
    if (r != DG_OK) return r;
    DG_HIP(hipEventRecord(c->step_ev[step % 2], s));
    return DG_OK;
  };
  static_assert(kAdaptiveLookahead == 1, "two step events in flight");
  *c->host_ndone = 0;
  for (int step = 0; step <= std::min(kAdaptiveLookahead, S - 1); ++step)
    if ((st = launch_step(step))) return st;
  for (int step = 0; step < S; ++step) {
    DG_HIP(hipEventSynchronize(c->step_ev[step % 2]));
    if ((st = take_status(c, "dg_denoise_block"))) return st;
    if (__atomic_load_n(c->host_ndone, __ATOMIC_ACQUIRE) >= B) break;
    const int next = step + 1 + kAdaptiveLookahead;
    if (next < S && (st = launch_step(next))) return st;
  }
  key.part = -2;
  return run_graph(c, key, s, [&](hipStream_t q) {
    return enqueue_block_end(c, cfg, B, kcs, vcs, Tmax, prefix_len, tokens_out, q);
  });
}

// After a block of dg_generate: an active row copies the block out, counts
// it and ends if it holds eos_id; a row that had ended undoes the block's
// prefix advance (it rode along).  One workgroup per row.
__global__ __launch_bounds__(256) void eos_block_kernel(
    const int32_t* __restrict__ blk_tokens, const int32_t* __restrict__ blk_steps, int L,
    int eos_id, int blk, int max_blocks, int32_t* __restrict__ active,
    int32_t* __restrict__ prefix_len, int32_t* __restrict__ tokens_out,
    int32_t* __restrict__ n_blocks, int32_t* __restrict__ steps_out) {
  const int b = blockIdx.x;
  if (!active[b]) {
    if (threadIdx.x == 0) prefix_len[b] -= L;
    return;
  }
  int hit = 0;
  for (int i = threadIdx.x; i < L; i += 256) {
    const int32_t t = blk_tokens[static_cast<size_t>(b) * L + i];
    tokens_out[(static_cast<size_t>(b) * max_blocks + blk) * L + i] = t;
    hit |= t == eos_id;
  }
  hit = __syncthreads_or(hit);
  if (threadIdx.x == 0) {
    n_blocks[b] = blk + 1;
    steps_out[static_cast<size_t>(b) * max_blocks + blk] = blk_steps[b];
    if (hit) active[b] = 0;
  }
}


}  // namespace

extern "C" {

size_t dg_ctx_workspace_size(const dg_model_dims* dims, int max_batch, int max_tokens,
                             int max_prefill_tokens) {
  if (!dims || max_batch <= 0 || max_tokens <= 0 || max_prefill_tokens < 0 ||
      max_prefill_tokens > (1 << 16) || check_dims(dims) != DG_OK)
    return 0;
  return layout(*dims, max_batch, max_tokens, max_prefill_tokens).total;
}

dg_status dg_ctx_create(dg_ctx** out, const dg_model_dims* dims, const dg_model_weights* w,
                        int max_batch, int max_tokens, int max_prefill_tokens, void* ws,
                        size_t ws_bytes) {
  set_error("");
  DG_CHECK_ARG(out && w, "dg_ctx_create: null pointer");
  dg_status st = check_dims(dims);
  if (st != DG_OK) return st;
  DG_CHECK_SHAPE(max_batch > 0 && max_batch < (1 << 24) && max_tokens > 0 && max_tokens <= 4096,
                 "dg_ctx_create: bad max_batch / max_tokens");
  DG_CHECK_SHAPE(max_prefill_tokens >= 0 && max_prefill_tokens <= (1 << 16),
                 "dg_ctx_create: max_prefill_tokens outside [0, 65536]");
  const int nl = dims->n_layers;
  DG_CHECK_ARG(w->emb && w->lm_head && w->wqkv && w->wo && w->wr && w->w_gate_up && w->w_down,
               "dg_ctx_create: null weight pointer");
  for (int l = 0; l < nl; ++l) {
    DG_CHECK_ARG(w->wqkv[l] && w->wo[l] && w->wr[l] && w->w_gate_up[l] && w->w_down[l],
                 "dg_ctx_create: null per-layer weight pointer");
    if (dims->expert_dtype == DG_FP8_E4M3)
      DG_CHECK_ARG(w->s_gate_up && w->s_down && w->s_gate_up[l] && w->s_down[l],
                   "dg_ctx_create: fp8 experts need scales");
  }
  const Layout L = layout(*dims, max_batch, max_tokens, max_prefill_tokens);
  if (!ws || ws_bytes < L.total) return fail(DG_ERR_WORKSPACE, "dg_ctx_create: workspace too small");
  int32_t* host_word = nullptr;     // [0] status, [1] stopped-row count
  DG_HIP(hipHostMalloc(reinterpret_cast<void**>(&host_word), 2 * sizeof(int32_t),
                       hipHostMallocMapped | hipHostMallocCoherent));
  host_word[0] = host_word[1] = 0;
  void* host_word_dev = nullptr;
  const hipError_t he = hipHostGetDevicePointer(&host_word_dev, host_word, 0);
  if (he != hipSuccess) {
    (void)hipHostFree(host_word);
    return fail(DG_ERR_HIP, std::string("dg_ctx_create: hipHostGetDevicePointer: ") +
                                hipGetErrorString(he));
  }
  hipStream_t cap = nullptr;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  hipError_t ce = hipStreamCreateWithFlags(&cap, hipStreamNonBlocking);
  if (ce == hipSuccess) ce = hipEventCreateWithFlags(&ev0, hipEventDisableTiming);
  if (ce == hipSuccess) ce = hipEventCreateWithFlags(&ev1, hipEventDisableTiming);
  if (ce != hipSuccess) {
    if (ev0) (void)hipEventDestroy(ev0);
    if (cap) (void)hipStreamDestroy(cap);
    (void)hipHostFree(host_word);
    return fail(DG_ERR_HIP, std::string("dg_ctx_create: stream / event: ") + hipGetErrorString(ce));
  }
  dg_ctx* c = new dg_ctx();
  c->host_status = host_word;
  c->host_status_dev = static_cast<int32_t*>(host_word_dev);
  c->host_ndone = host_word + 1;
  c->host_ndone_dev = static_cast<int32_t*>(host_word_dev) + 1;
  c->cap_stream = cap;
  c->step_ev[0] = ev0;
  c->step_ev[1] = ev1;
  c->d = *dims;
  c->emb = w->emb;
  c->lm = w->lm_head;
  for (int l = 0; l < nl; ++l) {
    c->wqkv.push_back(w->wqkv[l]);
    c->wo.push_back(w->wo[l]);
    c->wr.push_back(w->wr[l]);
    c->wgu.push_back(w->w_gate_up[l]);
    c->wd.push_back(w->w_down[l]);
    c->sgu.push_back(w->s_gate_up ? w->s_gate_up[l] : nullptr);
    c->sd.push_back(w->s_down ? w->s_down[l] : nullptr);
  }
  c->max_batch = max_batch;
  c->max_tokens = max_tokens;
  c->max_prefill = max_prefill_tokens;
  char* b = static_cast<char*>(ws);
  c->x = reinterpret_cast<float*>(b + L.x);
  c->h = b + L.h;
  c->qkv = b + L.qkv;
  c->attn_out = b + L.attn_out;
  c->router = reinterpret_cast<float*>(b + L.router);
  c->topk_ids = reinterpret_cast<int32_t*>(b + L.topk_ids);
  c->gates = reinterpret_cast<float*>(b + L.gates);
  c->offsets = reinterpret_cast<int32_t*>(b + L.offsets);
  c->sorted_rows = reinterpret_cast<int32_t*>(b + L.sorted_rows);
  c->attn_ws = b + L.attn_ws;
  c->moe_ws = b + L.moe_ws;
  c->logits = b + L.logits;
  c->samp_ws = b + L.samp_ws;
  c->tokens = reinterpret_cast<int32_t*>(b + L.tokens);
  c->committed = reinterpret_cast<uint8_t*>(b + L.committed);
  c->renoised = reinterpret_cast<uint8_t*>(b + L.renoised);
  c->maxprob = reinterpret_cast<float*>(b + L.maxprob);
  c->entropy = reinterpret_cast<float*>(b + L.entropy);
  c->mean_entropy = reinterpret_cast<float*>(b + L.mean_entropy);
  c->done = reinterpret_cast<int32_t*>(b + L.done);
  c->status = reinterpret_cast<int32_t*>(b + L.status);
  c->n_done = reinterpret_cast<int32_t*>(b + L.n_done);
  c->active = reinterpret_cast<int32_t*>(b + L.active);
  c->blk_tokens = reinterpret_cast<int32_t*>(b + L.blk_tokens);
  c->blk_steps = reinterpret_cast<int32_t*>(b + L.blk_steps);
  c->rope_tab = reinterpret_cast<float2*>(b + L.rope_tab);
  c->pending_tok = reinterpret_cast<int32_t*>(b + L.pending_tok);
  c->fused_tok = reinterpret_cast<int32_t*>(b + L.fused_tok);
  c->prefix_back = reinterpret_cast<int32_t*>(b + L.prefix_back);
  *out = c;
  return DG_OK;
}

dg_status dg_ctx_destroy(dg_ctx* ctx) {
  if (!ctx) return DG_OK;
  for (auto& kv : ctx->graphs) (void)hipGraphExecDestroy(kv.second);
  for (hipEvent_t e : ctx->step_ev)
    if (e) (void)hipEventDestroy(e);
  if (ctx->cap_stream) (void)hipStreamDestroy(ctx->cap_stream);
  if (ctx->host_status) (void)hipHostFree(ctx->host_status);
  delete ctx;
  return DG_OK;
}

dg_status dg_ctx_check_status(dg_ctx* ctx, void* stream) {
  set_error("");
  DG_CHECK_ARG(ctx != nullptr, "dg_ctx_check_status: ctx is null");
  DG_HIP(hipStreamSynchronize(static_cast<hipStream_t>(stream)));
  return take_status(ctx, "dg_ctx_check_status");
}

dg_status dg_ctx_set_graphs(dg_ctx* ctx, int use_graphs) {
  DG_CHECK_ARG(ctx != nullptr, "dg_ctx_set_graphs: ctx is null");
  ctx->use_graphs = use_graphs != 0;
  return DG_OK;
}

dg_status dg_ctx_set_router_override(dg_ctx* ctx, const float* const* logits, int n_tokens) {
  set_error("");
  DG_CHECK_ARG(ctx != nullptr, "dg_ctx_set_router_override: ctx is null");
  ctx->router_override.clear();
  ctx->router_override_tokens = 0;
  // captured graphs embed the routing inputs
  for (auto& kv : ctx->graphs) (void)hipGraphExecDestroy(kv.second);
  ctx->graphs.clear();
  if (!logits) return DG_OK;
  DG_CHECK_SHAPE(n_tokens > 0, "dg_ctx_set_router_override: n_tokens must be positive");
  for (int l = 0; l < ctx->d.n_layers; ++l)
    DG_CHECK_ARG(logits[l] != nullptr, "dg_ctx_set_router_override: null layer pointer");
  ctx->router_override.assign(logits, logits + ctx->d.n_layers);
  ctx->router_override_tokens = n_tokens;
  return DG_OK;
}

dg_status dg_model_forward(dg_ctx* ctx, const int32_t* tokens, float* x, int B, int n,
                           int layer_begin, int layer_end, void* const* k_caches,
                           void* const* v_caches, int Tmax, const int32_t* prefix_len,
                           int mask_mode, void* logits, void* stream) {
  set_error("");
  // token counts up to a prefill chunk (the activation buffers hold it)
  const int max_n = ctx ? std::max(ctx->max_tokens, B > 0 ? ctx->max_prefill / B : 0) : 0;
  dg_status st = check_run(ctx, B, n, k_caches, v_caches, Tmax, prefix_len, "dg_model_forward",
                           max_n);
  if (st != DG_OK || (st = check_no_pending(ctx, "dg_model_forward"))) return st;
  DG_CHECK_ARG(x != nullptr, "dg_model_forward: x is null");
  DG_CHECK_ARG(mask_mode == DG_MASK_CANVAS || mask_mode == DG_MASK_CAUSAL,
               "dg_model_forward: bad mask_mode");
  DG_CHECK_SHAPE(0 <= layer_begin && layer_begin <= layer_end && layer_end <= ctx->d.n_layers,
                 "dg_model_forward: bad layer range");
  DG_CHECK_SHAPE(!logits || layer_end == ctx->d.n_layers,
                 "dg_model_forward: logits need layer_end == n_layers");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t bytes = static_cast<size_t>(B) * n * ctx->d.d_model * 4;
  // the residual lives in the context workspace; x is the caller's view of it
  if (!tokens) DG_HIP(hipMemcpyAsync(ctx->x, x, bytes, hipMemcpyDeviceToDevice, s));
  if ((st = forward(ctx, tokens, B, n, layer_begin, layer_end, k_caches, v_caches, Tmax,
                    prefix_len, mask_mode, logits, false, s)))
    return st;
  DG_HIP(hipMemcpyAsync(x, ctx->x, bytes, hipMemcpyDeviceToDevice, s));
  return DG_OK;
}

dg_status dg_prefill(dg_ctx* ctx, const int32_t* prompt, int B, int n, void* const* k_caches,
                     void* const* v_caches, int Tmax, int32_t* prefix_len, void* stream) {
  set_error("");
  DG_CHECK_ARG(ctx && prompt, "dg_prefill: null pointer");
  DG_CHECK_SHAPE(n > 0 && n <= Tmax, "dg_prefill: n outside [1, Tmax]");
  DG_CHECK_SHAPE(B > 0 && B <= ctx->max_batch, "dg_prefill: B outside [1, max_batch]");
  // tokens per row of one chunk: the larger of the canvas limit and the
  // prefill limit shared by the rows
  const int chunk = std::max(ctx->max_tokens, ctx->max_prefill / B);
  dg_status st = check_run(ctx, B, std::min(n, chunk), k_caches, v_caches, Tmax, prefix_len,
                           "dg_prefill", chunk);
  if (st != DG_OK || (st = check_no_pending(ctx, "dg_prefill"))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the chunk's token ids, contiguous per row, staged in the canvas buffer
  for (int c0 = 0; c0 < n; c0 += chunk) {
    const int m = std::min(chunk, n - c0);
    DG_HIP(hipMemcpy2DAsync(ctx->tokens, m * sizeof(int32_t), prompt + c0, n * sizeof(int32_t),
                            m * sizeof(int32_t), B, hipMemcpyDeviceToDevice, s));
    if ((st = forward(ctx, ctx->tokens, B, m, 0, ctx->d.n_layers, k_caches, v_caches, Tmax,
                      prefix_len, DG_MASK_CAUSAL, nullptr, true, s)))
      return st;
    if ((st = launch_advance_prefix(prefix_len, B, m, s))) return st;
  }
  return DG_OK;
}

dg_status dg_ar_decode(dg_ctx* ctx, int B, int n_steps, const int32_t* tokens_in,
                       void* const* k_caches, void* const* v_caches, int Tmax,
                       int32_t* prefix_len, int32_t* tokens_out, void* stream) {
  set_error("");
  DG_CHECK_ARG(ctx && tokens_in && tokens_out, "dg_ar_decode: null pointer");
  DG_CHECK_SHAPE(n_steps >= 1 && n_steps <= Tmax, "dg_ar_decode: n_steps outside [1, Tmax]");
  DG_CHECK_SHAPE(ctx->d.vocab % 8 == 0, "dg_ar_decode: vocab must be a multiple of 8");
  dg_status st = check_run(ctx, B, 1, k_caches, v_caches, Tmax, prefix_len, "dg_ar_decode");
  if (st != DG_OK || (st = check_no_pending(ctx, "dg_ar_decode"))) return st;
  if ((st = take_status(ctx, "dg_ar_decode"))) return st;
  // graph key: F = -1 marks the AR loop (block keys have F >= 0)
  GraphKey key{B, Tmax, 1, n_steps, -1, 0.f, 0.f, 0.f, 0.f, 0.f, 0, 0, 0.f, 0, {}};
  for (int l = 0; l < ctx->d.n_layers; ++l) {
    key.ptrs.push_back(k_caches[l]);
    key.ptrs.push_back(v_caches[l]);
  }
  key.ptrs.push_back(prefix_len);
  key.ptrs.push_back(const_cast<int32_t*>(tokens_in));
  key.ptrs.push_back(tokens_out);
  return run_graph(ctx, key, static_cast<hipStream_t>(stream), [&](hipStream_t q) {
    return enqueue_ar(ctx, B, n_steps, tokens_in, k_caches, v_caches, Tmax, prefix_len,
                      tokens_out, q);
  });
}

dg_status dg_denoise_block(dg_ctx* ctx, const dg_sampler_cfg* cfg, int B, void* const* k_caches,
                           void* const* v_caches, int Tmax, int32_t* prefix_len,
                           int32_t* tokens_out, int32_t* steps_taken, void* stream) {
  set_error("");
  DG_CHECK_ARG(ctx && cfg && tokens_out && steps_taken, "dg_denoise_block: null pointer");
  dg_status st = check_block_cfg(cfg, "dg_denoise_block");
  if (st != DG_OK) return st;
  st = check_run(ctx, B, cfg->canvas_len, k_caches, v_caches, Tmax, prefix_len,
                 "dg_denoise_block");
  if (st != DG_OK || (st = check_no_pending(ctx, "dg_denoise_block"))) return st;
  if ((st = take_status(ctx, "dg_denoise_block"))) return st;
  return run_block(ctx, *cfg, B, k_caches, v_caches, Tmax, prefix_len, tokens_out, steps_taken,
                   static_cast<hipStream_t>(stream));
}

dg_status dg_denoise_block_deferred(dg_ctx* ctx, const dg_sampler_cfg* cfg, int B,
                                    void* const* k_caches, void* const* v_caches, int Tmax,
                                    int32_t* prefix_len, int32_t* tokens_out,
                                    int32_t* steps_taken, void* stream) {
  set_error("");
  const char* fn = "dg_denoise_block_deferred";
  DG_CHECK_ARG(ctx && cfg && tokens_out && steps_taken, std::string(fn) + ": null pointer");
  dg_status st = check_block_cfg(cfg, fn);
  if (st != DG_OK) return st;
  if (cfg->fixed_steps <= 0)
    return fail(DG_ERR_UNSUPPORTED, std::string(fn) + ": needs fixed_steps > 0");
  const int L = cfg->canvas_len;
  st = check_run(ctx, B, L, k_caches, v_caches, Tmax, prefix_len, fn);
  if (st != DG_OK) return st;
  // the fused first step runs 2L tokens per row: the activation and
  // attention buffers hold them when 2L fits the canvas or the prefill limit
  DG_CHECK_SHAPE(2 * L <= std::max(ctx->max_tokens, ctx->max_prefill / B),
                 std::string(fn) + ": needs 2 canvas_len <= max(max_tokens, max_prefill_tokens / B)");
  DG_CHECK_SHAPE(ctx->router_override.empty() || 2 * B * L <= ctx->router_override_tokens,
                 std::string(fn) + ": the router override must hold 2 B canvas_len tokens");
  DG_CHECK_SHAPE(Tmax >= 2 * L, std::string(fn) + ": Tmax smaller than two blocks");
  const std::vector<void*> ptrs = pending_key_ptrs(ctx, k_caches, v_caches, prefix_len);
  const bool fused = ctx->pending;
  if (fused)
    DG_CHECK_ARG(B == ctx->pending_B && L == ctx->pending_L && Tmax == ctx->pending_Tmax &&
                     ptrs == ctx->pending_ptrs,
                 std::string(fn) + ": the pending commit belongs to other caches or shapes");
  if ((st = take_status(ctx, fn))) return st;
  GraphKey key{B, Tmax, L, cfg->max_steps, cfg->fixed_steps, cfg->temp_start, cfg->temp_end,
               cfg->stop_entropy, cfg->commit_prob, cfg->renoise_prob, cfg->seed,
               cfg->commit_policy, cfg->entropy_bound, fused ? 11 : 10, ptrs};
  key.ptrs.push_back(tokens_out);
  key.ptrs.push_back(steps_taken);
  st = run_graph(ctx, key, static_cast<hipStream_t>(stream), [&](hipStream_t q) {
    return enqueue_block_deferred(ctx, *cfg, B, k_caches, v_caches, Tmax, prefix_len, tokens_out,
                                  steps_taken, fused, q);
  });
  if (st != DG_OK) return st;
  ctx->pending = true;
  ctx->pending_B = B;
  ctx->pending_L = L;
  ctx->pending_Tmax = Tmax;
  ctx->pending_ptrs = ptrs;
  return DG_OK;
}

dg_status dg_commit_pending(dg_ctx* ctx, int B, void* const* k_caches, void* const* v_caches,
                            int Tmax, const int32_t* prefix_len, void* stream) {
  set_error("");
  const char* fn = "dg_commit_pending";
  DG_CHECK_ARG(ctx != nullptr, std::string(fn) + ": ctx is null");
  if (!ctx->pending) return DG_OK;
  dg_status st = check_run(ctx, B, ctx->pending_L, k_caches, v_caches, Tmax, prefix_len, fn);
  if (st != DG_OK) return st;
  const std::vector<void*> ptrs = pending_key_ptrs(ctx, k_caches, v_caches, prefix_len);
  DG_CHECK_ARG(B == ctx->pending_B && Tmax == ctx->pending_Tmax && ptrs == ctx->pending_ptrs,
               std::string(fn) + ": the pending commit belongs to other caches or shapes");
  // graph key: F = -3 marks the commit of a deferred block
  GraphKey key{B, Tmax, ctx->pending_L, 0, -3, 0.f, 0.f, 0.f, 0.f, 0.f, 0, 0, 0.f, 0, ptrs};
  st = run_graph(ctx, key, static_cast<hipStream_t>(stream), [&](hipStream_t q) {
    return enqueue_commit_pending(ctx, B, ctx->pending_L, k_caches, v_caches, Tmax, prefix_len, q);
  });
  if (st != DG_OK) return st;
  ctx->pending = false;
  return DG_OK;
}

dg_status dg_generate(dg_ctx* ctx, const dg_sampler_cfg* cfg, int B, void* const* k_caches,
                      void* const* v_caches, int Tmax, int32_t* prefix_len, int32_t eos_id,
                      int max_blocks, int32_t* tokens_out, int32_t* n_blocks,
                      int32_t* steps_taken, void* stream) {
  set_error("");
  DG_CHECK_ARG(ctx && cfg && tokens_out && n_blocks && steps_taken, "dg_generate: null pointer");
  dg_status st = check_block_cfg(cfg, "dg_generate");
  if (st != DG_OK) return st;
  st = check_run(ctx, B, cfg->canvas_len, k_caches, v_caches, Tmax, prefix_len, "dg_generate");
  if (st != DG_OK || (st = check_no_pending(ctx, "dg_generate"))) return st;
  if ((st = take_status(ctx, "dg_generate"))) return st;
  const int L = cfg->canvas_len;
  DG_CHECK_SHAPE(max_blocks >= 1 && static_cast<int64_t>(max_blocks) * L <= Tmax,
                 "dg_generate: need 1 <= max_blocks and max_blocks * L <= Tmax");
  DG_CHECK_SHAPE(static_cast<int64_t>(B) * max_blocks * L < (1ll << 31),
                 "dg_generate: B * max_blocks * L too large");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int n_out = B * max_blocks * L;
  if ((st = fill_i32(tokens_out, n_out, -1, s))) return st;
  if ((st = fill_i32(n_blocks, B, 0, s))) return st;
  if ((st = fill_i32(steps_taken, B * max_blocks, 0, s))) return st;
  if ((st = fill_i32(ctx->active, B, 1, s))) return st;
  std::vector<int32_t> act(B);
  for (int blk = 0; blk < max_blocks; ++blk) {
    st = run_block(ctx, *cfg, B, k_caches, v_caches, Tmax, prefix_len, ctx->blk_tokens,
                   ctx->blk_steps, s);
    if (st != DG_OK) return st;
    eos_block_kernel<<<B, 256, 0, s>>>(ctx->blk_tokens, ctx->blk_steps, L, eos_id, blk,
                                       max_blocks, ctx->active, prefix_len, tokens_out, n_blocks,
                                       steps_taken);
    DG_LAUNCH_CHECK();
    DG_HIP(hipMemcpyAsync(act.data(), ctx->active, B * sizeof(int32_t), hipMemcpyDeviceToHost, s));
    DG_HIP(hipStreamSynchronize(s));
    if ((st = take_status(ctx, "dg_generate"))) return st;
    bool any = false;
    for (int b = 0; b < B; ++b) any = any || act[b] != 0;
    if (!any) break;
  }
  return DG_OK;
}

}  // extern "C"
