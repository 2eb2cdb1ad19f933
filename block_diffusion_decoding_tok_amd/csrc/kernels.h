// Internal launchers of libdg (host side).  Each launcher assumes its
// arguments were validated by the C ABI layer.
#pragma once

#include "common.h"

namespace dg {

// The adaptive block loop's step gate (see step_gate_closed): gated kernels
// skip their work once n_done[0] >= n; row_done[b] != 0 lets per-row kernels
// (attention) skip a row that has stopped.  Default: no gate.
struct StepGate {
  const int32_t* n_done = nullptr;
  int n = 0;
  const int32_t* row_done = nullptr;
};

// sampler.hip
size_t sampler_workspace_bytes(int B, int L, int V);
// api_sampler.cpp: host checks of dg_sampler_step's arguments (not the workspace)
dg_status check_sampler_step(const void* logits, int logit_dtype, int B, int L, int V, int step,
                             const dg_sampler_cfg* cfg, const int32_t* prefix_len,
                             const int32_t* tokens, const uint8_t* committed,
                             const uint8_t* renoised, const float* maxprob,
                             const float* entropy, const float* mean_entropy,
                             const int32_t* done);
// n_done (optional): incremented once by each row in the step that ends it.
dg_status launch_sampler(const void* logits, int logit_dtype, int B, int L, int V, int step,
                         const dg_sampler_cfg& cfg, const int32_t* prefix_len, int32_t* tokens,
                         uint8_t* committed, uint8_t* renoised, float* maxprob, float* entropy,
                         float* mean_entropy, int32_t* done, int32_t* status,
                         int32_t* steps_taken, void* ws, hipStream_t stream,
                         int32_t* n_done = nullptr);
dg_status launch_init_canvas(const int32_t* prefix_len, int B, int L, int V, uint64_t seed,
                             int32_t* tokens, uint8_t* committed, int32_t* done,
                             hipStream_t stream);
dg_status launch_philox(const uint32_t* ctr, int64_t n, uint64_t seed, uint32_t* out,
                        hipStream_t stream);
dg_status launch_gumbel(const uint32_t* w, int64_t n, float* out, hipStream_t stream);

// attention.hip
// Row strides (in elements) between consecutive tokens of q / k_new / v_new
// let the model pass slices of its fused QKV output.
struct AttnArgs {
  const void* q; const void* k_new; const void* v_new;
  int64_t q_stride, kv_stride;        // elements between tokens
  void* k_cache; void* v_cache;
  const int32_t* prefix_len;
  int B, Lq, Hq, Hkv, dh, Tmax, mask_mode;
  float rope_theta;
  int dtype;
  void* out;                          // [B, Lq, Hq, dh] dense
  int q_ready = 0;                    // q already rotated in the workspace, k/v in the caches
  int out_tiled = 0;                  // bf16 out in the tiled activation layout (xtile_offset)
  StepGate gate = {};
  // > 0: block-causal mask with groups of mask_blk tokens (a token sees the
  // cache and its block's tokens up to the end of its own group), in place
  // of mask_mode
  int mask_blk = 0;
};
// Scale of the packed q of the bf16 attention kernel: log2(e) / sqrt(dh), so
// that scores come out of the MFMA in the log2 domain.
inline float attn_q_scale(int dh) {
  return static_cast<float>(1.4426950408889634 / __builtin_sqrt(static_cast<double>(dh)));
}
size_t attention_workspace_bytes(int B, int Lq, int Hq, int Hkv, int dh, int Tmax, int dtype);
dg_status launch_attention(const AttnArgs& a, void* ws, hipStream_t stream);
dg_status launch_commit(const void* k_new, const void* v_new, int64_t kv_stride, void* k_cache,
                        void* v_cache, int32_t* prefix_len, int B, int L, int Hkv, int dh,
                        int Tmax, float rope_theta, int dtype, bool advance, hipStream_t stream);
dg_status launch_advance_prefix(int32_t* prefix_len, int B, int L, hipStream_t stream);

// moe.hip
size_t moe_route_workspace_bytes(int T, int E, int k);
dg_status launch_moe_route(const float* logits, int T, int E, int k, int32_t* topk_ids,
                           float* gates, int32_t* offsets, int32_t* sorted_rows, void* ws,
                           hipStream_t stream);
size_t moe_ffn_workspace_bytes(int T, int D, int I, int E, int k, int x_dtype);
// The expert FFN in three launches (gate/up, down, combine); launch_moe_ffn
// runs all three with h and y_slot carved from ws.
dg_status launch_moe_gate_up(const void* x, int x_dtype, const void* w_gate_up, int w_dtype,
                             int w_layout, const float* s_gate_up, const int32_t* offsets,
                             const int32_t* sorted_rows, int T, int D, int I, int E, int k,
                             void* h, hipStream_t stream, const StepGate& gate = {});
dg_status launch_moe_down(const void* h, int h_dtype, const void* w_down, int w_dtype,
                          int w_layout, const float* s_down, const float* gates,
                          const int32_t* offsets, const int32_t* sorted_rows, int T, int D, int I,
                          int E, int k, void* y_slot, hipStream_t stream,
                          const StepGate& gate = {});
dg_status launch_moe_combine(const void* y_slot, int dtype, int T, int D, int k, float* y,
                             hipStream_t stream);
// The intermediates launch_moe_ffn carves from its workspace.
void moe_ffn_workspace_split(void* ws, int T, int I, int k, int x_dtype, void** h,
                             void** y_slot);
dg_status launch_moe_ffn(const void* x, int x_dtype, const void* w_gate_up, const void* w_down,
                         int w_dtype, int w_layout, const float* s_gate_up, const float* s_down,
                         const int32_t* topk_ids, const float* gates, const int32_t* offsets,
                         const int32_t* sorted_rows, int T, int D, int I, int E, int k, float* y,
                         void* ws, hipStream_t stream);

// dense.hip: C = A W^T with A [M, K] (bf16 or f32), W [N, K] (same dtype,
// row-major or DG_LAYOUT_TILED for bf16), fp32 accumulation.  Epilogues: store
// in out_dtype, or add into f32 C.
enum GemmEpilogue { kStore = 0, kAccumulateF32 = 1 };
dg_status launch_gemm(const void* A, const void* W, void* C, int M, int N, int K, int dtype,
                      int w_layout, int out_dtype, GemmEpilogue ep, hipStream_t stream,
                      const StepGate& gate = {});
// The bf16 QKV projection with RoPE in its epilogue: q rotated and scaled
// into the attention workspace's packed q (its first bytes), k rotated and v
// into the caches at [P, P + Lq).  DG_ERR_UNSUPPORTED when the shape does not
// take the fused path (then run the projection and the attention's own RoPE).
// x_tiled: A in the tiled activation layout (tiled weights only).
struct QkvRope {
  const int32_t* prefix_len;
  int B, Lq, Hq, Hkv, dh, Tmax;
  float theta;
  void* q_out;
  void* k_cache;
  void* v_cache;
  int x_tiled;
  // (cos, sin) of every (token, pair) of the forward [B * Lq, dh / 2], as
  // RopeTable below writes it (the input RMSNorm of the layer)
  const float2* rope_tab;
};
bool qkv_rope_supported(const QkvRope& r, int K);
dg_status launch_qkv_rope(const void* A, const void* W, int K, int w_layout, const QkvRope& r,
                          hipStream_t stream, const StepGate& gate = {});
// C (=|+=) A W^T with A bf16 in the tiled activation layout and W tiled bf16
// (the O projection over more than 16 tokens); dense_xt_supported says which
// shapes run.
bool dense_xt_supported(int M, int N, int K);
dg_status launch_gemm_xt(const void* A, const void* W, void* C, int M, int N, int K,
                         int out_dtype, GemmEpilogue ep, hipStream_t stream,
                         const StepGate& gate = {});
// RMSNorm of f32 rows x [M, D] (eps 1e-6, unit gain) into out_dtype.
dg_status launch_rmsnorm(const float* x, void* out, int M, int D, int out_dtype,
                         hipStream_t stream);
// RoPE angles of a forward's tokens: with tab set, row t (token t % Lq of
// batch row t / Lq, position prefix_len[t / Lq] + t % Lq) also writes
// tab[t * pairs + j] = (cos, sin) of position * theta^(-2 j / (2 pairs)) for
// the pairs j < pairs, the angle reduced to [-pi, pi] in double first.
struct RopeTable {
  const int32_t* prefix_len = nullptr;
  int Lq = 1, pairs = 0;
  float theta = 0.f;
  float2* tab = nullptr;
};
// Rows of a norm that reads a subset of x: with blk > 0, output row r reads
// input row (r / blk) * in_blk + in_off + r % blk (e.g. the last L of every
// 2L-token row of a forward); blk == 0: output row r reads row r.
struct NormRows {
  int blk = 0, in_blk = 0, in_off = 0;
};
// The MoE combine fused into the next RMSNorm: x[t] += sum_j y_slot[t * k + j]
// (slot order, as launch_moe_combine), then out = RMSNorm(x).  y_slot may be
// null (plain RMSNorm); slot_dtype is DG_BF16 or DG_F32.  out_tiled: bf16
// out in the tiled activation layout (D % 64 == 0, D <= 4096).  rope: the
// RoPE table of the rows (pairs <= 256), written alongside.  rows: M output
// rows read (and combine into) the input rows NormRows maps them to.
dg_status launch_combine_rmsnorm(const void* y_slot, int slot_dtype, int k, float* x, void* out,
                                 int M, int D, int out_dtype, hipStream_t stream,
                                 bool out_tiled = false, const RopeTable& rope = {},
                                 const NormRows& rows = {});
// x[t] = emb[tokens[t]] as f32.
dg_status launch_embed(const int32_t* tokens, const void* emb, float* x, int M, int D,
                       int dtype, hipStream_t stream);

// init.hip
dg_status launch_fill_normal(void* dst, int dtype, size_t n, float std, uint64_t seed,
                             uint32_t stream_id, hipStream_t stream);
dg_status launch_quantize_fp8_rows(const float* src, uint8_t* q, float* scale, int64_t rows,
                                   int cols, hipStream_t stream);
dg_status launch_pack_weights(const void* src, void* dst, int64_t groups, int N, int K,
                              int elem_bytes, hipStream_t stream);
dg_status launch_quantize_mxfp4(const float* src, uint8_t* codes, uint8_t* scales, int64_t n,
                                hipStream_t stream);
dg_status launch_pack_mxfp4(const uint8_t* codes, const uint8_t* scales, void* dst,
                            int64_t groups, int N, int K, hipStream_t stream);

}  // namespace dg
