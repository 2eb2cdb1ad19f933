/*
 * dg.h -- C ABI of libdg.so: the canvas denoising step of a block-
 * autoregressive, uniform-state text-diffusion decoder on MI355X (gfx950).
 *
 * Pages cited (by title; sections are the pages' own headings):
 *   [TR]    "[AI] DiffusionGemma: 256토큰 블록을 병렬 정제하는 확산 LLM"
 *           (summary of the DiffusionGemma technical report)
 *   [GUIDE] aisparkup "diffusion-gemma tutorial / developer guide"
 *   [GN]    "DiffusionGemma: 4배 빠른 텍스트 생성" (GeekNews)
 *   [WE0]   test.we0.ai article on DiffusionGemma
 *   [JPH]   "구글, 순차 처리 탈피한 확산 기반 AI 모델 디퓨전젬마 공개"
 *
 * Conventions for every entry point
 *   - All tensor arguments are DEVICE pointers owned by the caller, row-major,
 *     densely packed in the order of the dimensions given.  Arrays of per-layer
 *     pointers (``void* const*``) are HOST arrays of device pointers.
 *   - ``stream`` is a hipStream_t (NULL = the default stream).  Every call is
 *     asynchronous on that stream; results are valid once it is synchronized.
 *     Nothing is allocated per call: the caller passes a workspace of at least
 *     the size returned by the matching *_workspace_size() function.
 *   - Arguments are validated on the host before anything is launched; an
 *     invalid call returns a negative dg_status and launches nothing.  The
 *     message of the last failure on the calling thread is dg_last_error().
 *   - Device-side conditions (non-finite logits) are reported through a
 *     caller-provided device status word (see dg_sampler_step); the decoder
 *     calls report them as DG_ERR_NONFINITE (see dg_ctx_check_status).
 */
#ifndef DG_H_
#define DG_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DG_OK = 0,
  DG_ERR_INVALID_ARG = -1,   /* null pointer, bad enum, negative size */
  DG_ERR_SHAPE = -2,         /* sizes inconsistent or outside supported set */
  DG_ERR_UNSUPPORTED = -3,   /* valid but not implemented combination */
  DG_ERR_WORKSPACE = -4,     /* workspace missing or too small */
  DG_ERR_HIP = -5,           /* a HIP runtime call failed (see dg_last_error) */
  DG_ERR_NONFINITE = -6      /* NaN / Inf logits met by a decoder call (see dg_ctx_check_status) */
} dg_status;

/* DG_MXFP4: OCP Microscaling MXFP4 (FP4 E2M1 elements, blocks of 32 along K
 * sharing one E8M0 scale 2^(e - 127)); expert weights only, tile-packed with
 * their scales (see dg_layout; the 4-bit counterpart of the NVFP4 weights the
 * GeekNews page's "최적화와 실행 환경" names). */
typedef enum { DG_F32 = 0, DG_BF16 = 1, DG_FP8_E4M3 = 2 /* OCP e4m3fn */, DG_MXFP4 = 3 } dg_dtype;

typedef enum { DG_MASK_CANVAS = 0, DG_MASK_CAUSAL = 1 } dg_mask_mode;

/* Weight layouts for [G, N, K] weight tensors (G groups, e.g. experts).
 *   DG_LAYOUT_ROWMAJOR  element (g, n, k) at (g * N + n) * K + k.
 *   DG_LAYOUT_TILED     blocks of 16 rows x 64 k.  One matrix (G = 1): block
 *                       (n / 16, k / 64) at (n / 16 * K / 64 + k / 64) * 1024
 *                       elements (a 16-row tile contiguous).  A stack of G > 1
 *                       (experts): block (g, n / 16, k / 64) at
 *                       ((k / 64 * G + g) * N / 16 + n / 16) * 1024 elements
 *                       (the k chunk of every expert's tiles together, so the
 *                       waves streaming different experts read neighbouring
 *                       addresses); inside a block, with r = n % 16, q = (k % 64) / 16:
 *                       1-byte types: lane = r + 16 q holds k % 16 at lane * 16;
 *                       2-byte types: half h = (k % 16) / 8 at h * 512 + lane * 8.
 *                       It is the order in which a 64-lane wave loads an MFMA
 *                       A-operand tile, so every load reads 1 KB contiguous.
 *                       Needs N % 16 == 0 and K % 64 == 0 (dg_pack_weights).
 *   DG_MXFP4 weights are always tile-packed (dg_pack_mxfp4), in blocks of
 *   16 rows x 64 k of 544 bytes, block (g, n / 16, k / 64) at byte
 *   ((g * N / 16 + n / 16) * K / 64 + k / 64) * 544; inside a block, with
 *   r = n % 16, q = (k % 64) / 16: bytes 8 (r + 16 q) .. +7 hold the codes of
 *   k % 64 = 16 q .. 16 q + 15 (two per byte, the lower k in the low nibble),
 *   byte 512 + 16 h + r the E8M0 scale of row r, k % 64 in [32 h, 32 h + 32).
 *   A tensor [G, N, K] takes G * N * K * 17 / 32 bytes. */
typedef enum { DG_LAYOUT_ROWMAJOR = 0, DG_LAYOUT_TILED = 1 } dg_layout;

/* Device status-word bits. */
#define DG_STATUS_NONFINITE_LOGITS 1

/*
 * Sampler settings.  [TR] section "DiffusionGemma의 구성" (sampler settings):
 * canvas length 256, at most 48 denoising steps, temperature linear from 0.8 to
 * 0.4, adaptive stop threshold 0.005.  The commit / re-noise probabilities
 * (0.9 / 0.1) are not given by the pages.
 *   canvas_len    L, tokens per block
 *   max_steps     S, step cap; the temperature schedule runs over S
 *   fixed_steps   0 = adaptive stop; F > 0 = exactly F steps, no stop test
 *   seed          Philox4x32-10 key (lo, hi words)
 *   commit_policy DG_COMMIT_MAXPROB: an uncommitted position commits when its
 *                 maxprob >= commit_prob.  DG_COMMIT_ENTROPY_BOUND: the
 *                 serving configuration's "entropy_bound" sampler (developer
 *                 guide, "vLLM으로 서빙하기": bound 0.1, a confidence-based
 *                 early exit), read as entropy-bounded unmasking: the
 *                 uncommitted positions ranked by (entropy, position), the
 *                 longest prefix whose entropies sum, minus their maximum, to
 *                 at most entropy_bound commits (at least one per step); in
 *                 the adaptive mode the block also ends when all committed.
 *   entropy_bound the bound in nats (>= 0), DG_COMMIT_ENTROPY_BOUND only
 */
typedef enum { DG_COMMIT_MAXPROB = 0, DG_COMMIT_ENTROPY_BOUND = 1 } dg_commit_policy;
typedef struct {
  int32_t canvas_len;
  int32_t max_steps;
  int32_t fixed_steps;
  float temp_start;
  float temp_end;
  float stop_entropy;
  float commit_prob;
  float renoise_prob;
  uint64_t seed;
  int32_t commit_policy;
  float entropy_bound;
} dg_sampler_cfg;

/* Library version (major * 10000 + minor * 100 + patch). */
int dg_version(void);
/* Message of the last failing call on this thread ("" if none). */
const char* dg_last_error(void);

/* ------------------------------------------------------------------ sampler
 * dg_sampler_step: one step of the canvas sampler over B rows.
 * Defines: [TR] "DiffusionGemma의 구성" (temperature schedule, step cap, stop
 * threshold); [GUIDE] "Uniform State Diffusion" (confident tokens anchor,
 * unconfident ones are re-randomized); [GN] "텍스트 확산의 작동 방식".
 *   T_s = temp_start + (temp_end - temp_start) * step / (max_steps - 1)
 *   per position: z = logits / T_s; maxprob = max softmax(z); entropy (nats);
 *   sample = argmax_v (z_v + Gumbel_v) with Gumbel from Philox4x32-10 counter
 *   (v >> 2, prefix_len[b] + i, step, b), lane v & 3 (ties -> lowest v).
 *   mean_entropy[b] = mean over all L positions; the step ends the row if
 *   fixed_steps ? step == fixed_steps - 1 : (mean < stop_entropy || step ==
 *   max_steps - 1).  For uncommitted positions: maxprob >= commit_prob ->
 *   token = sample, committed = 1; else maxprob < renoise_prob and the step
 *   does not end the row -> token = uniform id from counter (0, pos, step,
 *   (1 << 24) | b), renoised = 1; else token = sample.  done[b] = ends.
 * Arguments
 *   logits     [B, L, V] DG_BF16 or DG_F32 (logit_dtype); V % 8 == 0, V < 2^31
 *   prefix_len [B] int32: absolute position of canvas slot 0
 *   tokens, committed [B, L] in/out; renoised, maxprob, entropy [B, L] out;
 *   mean_entropy [B] out; done [B] in/out (rows with done = 1 on entry are not
 *   touched at all, outputs included)
 *   status     optional int32 device word: DG_STATUS_NONFINITE_LOGITS is OR-ed
 *              in when a processed row holds a NaN/Inf logit
 *   ws         >= dg_sampler_workspace_size(B, L, V) bytes
 * Errors: DG_ERR_INVALID_ARG (null pointer, bad dtype), DG_ERR_SHAPE (sizes,
 * step outside [0, max_steps) or [0, fixed_steps)), DG_ERR_WORKSPACE.
 */
size_t dg_sampler_workspace_size(int B, int L, int V);
dg_status dg_sampler_step(const void* logits, int logit_dtype, int B, int L, int V,
                          int step, const dg_sampler_cfg* cfg, const int32_t* prefix_len,
                          int32_t* tokens, uint8_t* committed, uint8_t* renoised,
                          float* maxprob, float* entropy, float* mean_entropy,
                          int32_t* done, int32_t* status, void* ws, size_t ws_bytes,
                          void* stream);

/* dg_sampler_step_noalloc: dg_sampler_step for callers that cannot allocate
 * device memory or pass a workspace (code under hipGraph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Same arguments, results
 * and errors as dg_sampler_step, without ws / ws_bytes: the workspace is a
 * library-owned device array of DG_SAMPLER_SCRATCH_BYTES on each GPU the call
 * runs on (held until the process ends).  Calls with
 * dg_sampler_workspace_size(B, L, V) > DG_SAMPLER_SCRATCH_BYTES (e.g. more
 * than 2048 positions at V = 2^18) return DG_ERR_WORKSPACE and launch
 * nothing.  It allocates nothing.  Every call on a GPU shares that GPU's
 * array: calls that overlap on one GPU (several streams, several host
 * threads) race and must be serialized by the caller. */
#define DG_SAMPLER_SCRATCH_BYTES (1u << 20)
dg_status dg_sampler_step_noalloc(const void* logits, int logit_dtype, int B, int L, int V,
                                  int step, const dg_sampler_cfg* cfg, const int32_t* prefix_len,
                                  int32_t* tokens, uint8_t* committed, uint8_t* renoised,
                                  float* maxprob, float* entropy, float* mean_entropy,
                                  int32_t* done, int32_t* status, void* stream);

/* dg_init_canvas: the block's starting canvas ([GN] "텍스트 확산의 작동 방식";
 * [GUIDE] "Uniform State Diffusion": random placeholder tokens).
 * tokens[b, i] = uniform id in [0, V) from Philox counter
 * (0, prefix_len[b] + i, 0, (2 << 24) | b); committed = 0; done = 0.
 *   prefix_len [B] int32; tokens [B, L] int32; committed [B, L] u8; done [B]. */
dg_status dg_init_canvas(const int32_t* prefix_len, int B, int L, int V, uint64_t seed,
                         int32_t* tokens, uint8_t* committed, int32_t* done, void* stream);

/* ---------------------------------------------------------------- attention
 * dg_canvas_attention: attention of a block of Lq queries per row over the
 * cached prefix plus the block itself.  Every canvas position sees every
 * other ([GN] "핵심 트레이드오프"; [WE0] "양방향 어텐션과 자기 수정의 역할") and
 * the prefix from the KV cache ([GUIDE] "Block Autoregressive Diffusion"); the
 * prompt never sees the canvas ([TR] "DiffusionGemma의 구성", block-diagonal
 * mask).  Scores q.k / sqrt(dh); query head h reads KV head h / (Hq / Hkv);
 * RoPE (pairs j, j + dh/2, angle pos * theta^(-2j/dh)) at absolute positions
 * P_b + i rotates q and k_new.  Mode CANVAS: query i sees keys [0, P_b + Lq);
 * mode CAUSAL: keys [0, P_b + i].  The rotated k_new and v_new are written to
 * cache slots [P_b, P_b + Lq); prefix_len is NOT advanced.
 *   q        [B, Lq, Hq, dh]      k_new, v_new [B, Lq, Hkv, dh] (k un-rotated)
 *   k_cache, v_cache [B, Hkv, Tmax, dh], slots [0, P_b) hold rotated keys
 *   prefix_len [B] int32 device; requires P_b + Lq <= Tmax (not checked on the
 *   device: the caller guarantees it)
 *   out      [B, Lq, Hq, dh]
 *   dtype    DG_BF16 (MFMA path, fp32 accumulation) or DG_F32
 *   dh in {16, 64, 128} for DG_F32 and dh == 128 for DG_BF16; Hq % Hkv == 0.
 */
size_t dg_attention_workspace_size(int B, int Lq, int Hq, int Hkv, int dh, int Tmax, int dtype);
dg_status dg_canvas_attention(const void* q, const void* k_new, const void* v_new,
                              void* k_cache, void* v_cache, const int32_t* prefix_len,
                              int B, int Lq, int Hq, int Hkv, int dh, int Tmax,
                              int mask_mode, float rope_theta, int dtype, void* out,
                              void* ws, size_t ws_bytes, void* stream);

/* dg_commit_block: commit a finished block to the KV cache ([TR]
 * "DiffusionGemma의 구성", flowchart; [GUIDE] "Block Autoregressive Diffusion";
 * [WE0] "DiffusionGemma가 다르게 하는 점").  Rotates k_new at positions
 * P_b + i, writes k and v_new to cache slots [P_b, P_b + L), then
 * prefix_len[b] += L.  Same layouts and dtypes as dg_canvas_attention.  The
 * caller guarantees P_b + L <= Tmax. */
dg_status dg_commit_block(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                          int32_t* prefix_len, int B, int L, int Hkv, int dh, int Tmax,
                          float rope_theta, int dtype, void* stream);

/* ---------------------------------------------------------------------- MoE
 * dg_moe_route: top-k routing of T tokens over E experts ([WE0] "26B MoE 설계가
 * 의미하는 것": only selected experts run).  Order: logit descending, ties to
 * the lower expert id; gates = softmax of the k selected logits;
 * expert_offsets = exclusive prefix sum of per-expert counts; sorted_rows = the
 * slot entries t * k + j ordered stably by expert.
 *   router_logits [T, E] f32; topk_ids [T, k] i32; gates [T, k] f32;
 *   expert_offsets [E + 1] i32; sorted_rows [T * k] i32.
 *   E <= 256, k <= min(E, 16), T * k < 2^31.  ws >= dg_moe_route_workspace_size.
 */
size_t dg_moe_route_workspace_size(int T, int E, int k);
dg_status dg_moe_route(const float* router_logits, int T, int E, int k, int32_t* topk_ids,
                       float* gates, int32_t* expert_offsets, int32_t* sorted_rows,
                       void* ws, size_t ws_bytes, void* stream);

/* dg_moe_ffn: y[t] += sum_j gates[t, j] * FFN_{topk_ids[t, j]}(x[t]) with
 * FFN_e(u) = (GELU_erf(u Wg_e^T) * (u Wu_e^T)) Wd_e^T, summed in slot order.
 *   x          [T, D] DG_BF16 (with DG_BF16 / DG_FP8_E4M3 / DG_MXFP4 weights)
 *              or DG_F32 (with DG_F32 weights)
 *   w_gate_up  [E, 2I, D]: rows 0..I-1 gate, I..2I-1 up;  w_down [E, D, I];
 *              in w_layout (DG_LAYOUT_TILED only with DG_BF16 / DG_FP8_E4M3;
 *              DG_MXFP4 weights must be DG_LAYOUT_TILED: the tiled MXFP4
 *              layout with the block scales inside, from dg_pack_mxfp4)
 *   s_gate_up  [E, 2I], s_down [E, D] f32 per-row scales (DG_FP8_E4M3 only;
 *              the weight is byte value * scale); ignored otherwise
 *   routing tables as produced by dg_moe_route; y [T, D] f32, accumulated.
 *   D % 128 == 0 and I % 64 == 0 for the bf16 / fp8 (MFMA) paths.
 * ws >= dg_moe_ffn_workspace_size(T, D, I, E, k, x_dtype).  It runs the three
 * steps below (gate/up, down, combine) with h and y_slot carved from ws. */
size_t dg_moe_ffn_workspace_size(int T, int D, int I, int E, int k, int x_dtype);
dg_status dg_moe_ffn(const void* x, int x_dtype, const void* w_gate_up, const void* w_down,
                     int w_dtype, int w_layout, const float* s_gate_up, const float* s_down,
                     const int32_t* topk_ids, const float* gates, const int32_t* expert_offsets,
                     const int32_t* sorted_rows, int T, int D, int I, int E, int k, float* y,
                     void* ws, size_t ws_bytes, void* stream);

/* The expert FFN of dg_moe_ffn as its three steps ([WE0] "26B MoE 설계가
 * 의미하는 것": each token runs only its selected experts), for callers that
 * schedule or time them apart.  Arguments, dtypes, layouts and limits as in
 * dg_moe_ffn; the intermediates are dense device arrays owned by the caller.
 *
 * dg_moe_gate_up: for every sorted position p of expert e (expert_offsets[e]
 *   <= p < expert_offsets[e + 1]) and token t = sorted_rows[p] / k,
 *   h[p, :] = GELU_erf(x[t] Wg_e^T) * (x[t] Wu_e^T).
 *   h [T * k, I] in x_dtype.
 * dg_moe_down: for every sorted position p, slot s = sorted_rows[p],
 *   y_slot[s, :] = gates[s] * (h[p] Wd_e^T).  h_dtype is x_dtype of the
 *   gate/up step; y_slot [T * k, D] in h_dtype.
 * dg_moe_combine: y[t, :] += sum_{j < k} y_slot[t * k + j, :] in slot order.
 *   y_slot in dtype (DG_BF16 or DG_F32); y [T, D] f32.  D % 4 == 0. */
dg_status dg_moe_gate_up(const void* x, int x_dtype, const void* w_gate_up, int w_dtype,
                         int w_layout, const float* s_gate_up, const int32_t* expert_offsets,
                         const int32_t* sorted_rows, int T, int D, int I, int E, int k, void* h,
                         void* stream);
dg_status dg_moe_down(const void* h, int h_dtype, const void* w_down, int w_dtype, int w_layout,
                      const float* s_down, const float* gates, const int32_t* expert_offsets,
                      const int32_t* sorted_rows, int T, int D, int I, int E, int k, void* y_slot,
                      void* stream);
dg_status dg_moe_combine(const void* y_slot, int dtype, int T, int D, int k, float* y,
                         void* stream);

/* ----------------------------------------------------------- whole decoder
 * A random-init decoder of n_layers pre-norm layers: RMSNorm (eps 1e-6, unit
 * gain) -> fused QKV -> canvas attention -> O projection + residual -> RMSNorm
 * -> router -> top-k MoE + residual; final RMSNorm -> untied LM head.  Dense
 * weights and activations use act_dtype (DG_BF16 or DG_F32); experts use
 * expert_dtype (DG_BF16, DG_FP8_E4M3, DG_MXFP4 with the tiled layout, or
 * DG_F32 with DG_F32 activations).  The residual stream is f32.  Weight shapes: emb, lm_head [V, D]; wqkv
 * [(Hq + 2 Hkv) dh, D] (rows q | k | v); wo [D, Hq dh]; wr [E, D]; experts as
 * in dg_moe_ffn.  emb is always row-major; every other weight is in
 * weight_layout (DG_LAYOUT_TILED only with bf16 activations).  KV caches: per
 * layer [B, Hkv, Tmax, dh] in act_dtype.
 */
typedef struct {
  int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim;
  int32_t n_experts, top_k, d_ff, vocab;
  float rope_theta;
  int32_t act_dtype;
  int32_t expert_dtype;
  int32_t weight_layout;
} dg_model_dims;

typedef struct {
  const void* emb;
  const void* lm_head;
  const void* const* wqkv;        /* host array [n_layers] of device pointers */
  const void* const* wo;
  const void* const* wr;
  const void* const* w_gate_up;
  const void* const* w_down;
  const float* const* s_gate_up;  /* NULL entries allowed unless fp8 */
  const float* const* s_down;
} dg_model_weights;

typedef struct dg_ctx dg_ctx;

/* Workspace for a context serving up to max_batch rows of max_tokens tokens
 * per forward (the canvas length, the AR and model-forward limit) and prefill
 * forwards of up to max_prefill_tokens tokens over all rows (a row's prefill
 * chunk is max(max_tokens, max_prefill_tokens / B) tokens; 0: chunks of
 * max_tokens).  Only the activation buffers grow with max_prefill_tokens
 * (about 80 KB per token at the decoder's full width), not the logits and
 * sampler buffers.  max_prefill_tokens <= 65536.  0 on invalid input. */
size_t dg_ctx_workspace_size(const dg_model_dims* dims, int max_batch, int max_tokens,
                             int max_prefill_tokens);
/* Creates a context holding the dims, copies of the weight pointers (not the
 * weights) and the workspace pointer; the caller keeps every buffer alive.
 * Also allocates the context's own small host state: a pinned host word
 * pair (status and stopped-row count), a capture stream and two events. */
dg_status dg_ctx_create(dg_ctx** out, const dg_model_dims* dims, const dg_model_weights* w,
                        int max_batch, int max_tokens, int max_prefill_tokens, void* ws,
                        size_t ws_bytes);
dg_status dg_ctx_destroy(dg_ctx* ctx);
/* use_graphs != 0 (default): dg_denoise_block replays a captured hipGraph. */
dg_status dg_ctx_set_graphs(dg_ctx* ctx, int use_graphs);
/* Non-finite logits (the failure the sampler and the AR argmax detect: a NaN
 * or Inf anywhere in a row's logits) in the decoder calls.  Each block and
 * each AR run clears the context's device status word when it starts; the
 * sampler steps (and the AR argmax) OR in DG_STATUS_NONFINITE_LOGITS; the end
 * of the block (of each adaptive chunk, of the AR run) stores a non-zero word
 * into a host-visible word of the context (pinned host memory, allocated by
 * dg_ctx_create).  Every decoder call (dg_denoise_block, dg_generate,
 * dg_ar_decode) first takes that word: if it is set, the call clears it and
 * returns DG_ERR_NONFINITE without launching anything.  Calls that wait on
 * the stream anyway (the adaptive mode after each chunk, dg_generate after
 * each block) return DG_ERR_NONFINITE as soon as they see it, leaving the
 * block uncommitted (prefix_len not advanced).  An asynchronous call (fixed
 * steps with graphs, dg_ar_decode) returns DG_OK and its non-finite logits
 * are reported by the next call on the context that runs after the device
 * finished it, or by dg_ctx_check_status.
 * dg_ctx_check_status: waits for stream, then returns DG_ERR_NONFINITE (and
 * clears the word) if a finished call met non-finite logits, else DG_OK. */
dg_status dg_ctx_check_status(dg_ctx* ctx, void* stream);
/* Benchmarking hook: route every forward with caller-supplied router logits
 * instead of the router projection's output (the projection still runs).
 * logits: host array [n_layers] of device pointers to f32 [n_tokens, E]; a
 * forward over B * n tokens uses the first B * n rows (requires B * n <=
 * n_tokens).  NULL restores the model's own routing.  Lets a random-init model
 * run with a stated routing distribution (e.g. a planted hot-expert skew)
 * instead of the one its random weights produce. */
dg_status dg_ctx_set_router_override(dg_ctx* ctx, const float* const* logits, int n_tokens);

/* dg_model_forward: one forward over n tokens per row (n <= max(max_tokens,
 * max_prefill_tokens / B)) at cache positions [P_b, P_b + n).  If tokens != NULL the residual x is first set to the
 * embeddings; layers [layer_begin, layer_end) are applied to x [B * n, D] f32
 * in place (each writes its rotated K/V to its cache at [P_b, P_b + n)); if
 * logits != NULL (requires layer_end == n_layers) the final RMSNorm + LM head
 * writes logits [B, n, V] in act_dtype.  prefix_len is not advanced. */
dg_status dg_model_forward(dg_ctx* ctx, const int32_t* tokens, float* x, int B, int n,
                           int layer_begin, int layer_end, void* const* k_caches,
                           void* const* v_caches, int Tmax, const int32_t* prefix_len,
                           int mask_mode, void* logits, void* stream);

/* dg_prefill: encode a prompt into the KV cache ([TR] "DiffusionGemma의 구성",
 * flowchart: prompt -> KV cache; [GUIDE] "vLLM으로 서빙하기": chunked
 * prefill) with a causal mask, in chunks of max(max_tokens,
 * max_prefill_tokens / B) tokens per row (large chunks stream each layer's
 * expert weights once per chunk instead of once per canvas-sized chunk),
 * starting at prefix_len[b] and advancing it by n.  prompt [B, n] i32. */
dg_status dg_prefill(dg_ctx* ctx, const int32_t* prompt, int B, int n, void* const* k_caches,
                     void* const* v_caches, int Tmax, int32_t* prefix_len, void* stream);

/* dg_denoise_block: one whole block ([TR] "DiffusionGemma의 구성", flowchart;
 * [GUIDE] "Block Autoregressive Diffusion"): init canvas; per step a forward
 * over the canvas (canvas mask), the LM head and dg_sampler_step, until every
 * row is done (adaptive) or fixed_steps; then one more forward of the final
 * tokens commits every layer's K/V to slots [P_b, P_b + L) and prefix_len += L.
 *   tokens_out [B, L] i32; steps_taken [B] i32 (steps each row ran).
 *   requires B <= max_batch, L <= max_tokens, P_b + L <= Tmax.
 * With fixed_steps the block is one asynchronous hipGraph (graphs on).  In
 * the adaptive mode each step is its own graph: the sampler counts the rows
 * that stopped on the device, and every heavy kernel of a step (projections,
 * attention -- also per stopped row --, experts, LM head, sampler) returns
 * at once when that count equals B.  The host keeps one step queued beyond
 * the step it waits for (an event per step, no stream synchronization) and
 * reads the count from a host-visible word after that step; once every row
 * stopped it queues the commit, so at most one step after the end runs, and
 * that one gated.  The call returns once the commit is queued.  Non-finite
 * logits: DG_ERR_NONFINITE, as described at dg_ctx_check_status. */
dg_status dg_denoise_block(dg_ctx* ctx, const dg_sampler_cfg* cfg, int B, void* const* k_caches,
                           void* const* v_caches, int Tmax, int32_t* prefix_len,
                           int32_t* tokens_out, int32_t* steps_taken, void* stream);

/* dg_generate: EOS-terminated multi-block decode ([TR] "DiffusionGemma의
 * 구성", flowchart: after each committed block, stop at EOS, else start the
 * next canvas).  Blocks as in dg_denoise_block, one after another; a row ends
 * after the first block holding eos_id, or after max_blocks blocks.  Rows
 * that ended ride along in later blocks with prefix_len frozen (their cache
 * slots past the prefix are scratch).  The call waits on the stream after
 * each block and returns when every row ended.
 *   tokens_out [B, max_blocks, L] i32 (-1 after a row's last block);
 *   n_blocks [B] i32 (blocks each row produced); steps_taken [B, max_blocks]
 *   i32 (0 after a row's last block); requires P_b + max_blocks * L <= Tmax. */
dg_status dg_generate(dg_ctx* ctx, const dg_sampler_cfg* cfg, int B, void* const* k_caches,
                      void* const* v_caches, int Tmax, int32_t* prefix_len, int32_t eos_id,
                      int max_blocks, int32_t* tokens_out, int32_t* n_blocks,
                      int32_t* steps_taken, void* stream);

/* dg_denoise_block_deferred: dg_denoise_block (fixed_steps > 0 only) with its
 * commit forward deferred into the next block ([TR] "DiffusionGemma의 구성",
 * flowchart: a finished block enters the KV cache before the next block
 * denoises).  At the end the block's final tokens become the context's
 * pending block: tokens_out is written and prefix_len += L as with
 * dg_denoise_block, but the cache slots [P_b - L, P_b) do not hold the final
 * tokens' K/V yet.  The next dg_denoise_block_deferred (same B, L, Tmax,
 * caches and prefix_len array) runs its first step as one forward over each
 * row's pending block (positions [P_b - L, P_b)) followed by its new canvas
 * ([P_b, P_b + L)) with a block-causal mask: the pending block attends to the
 * cache before it and to itself, exactly as its commit forward would (and
 * writes the same K/V), the canvas to the cache, the pending block and
 * itself, as its first step would; logits are taken for the canvas rows
 * only.  Each layer's expert weights then stream once for both.  The last
 * pending block is committed by dg_commit_pending.  While a commit is pending
 * every other decoder call on the context (dg_model_forward, dg_prefill,
 * dg_ar_decode, dg_denoise_block, dg_generate) fails with DG_ERR_INVALID_ARG.
 *   requires 2 L <= max(max_tokens, max_prefill_tokens / B) (the fused step's
 *   2L tokens per row), Tmax >= 2 L, and a router override (if set) of at
 *   least 2 B L tokens.  Errors: DG_ERR_UNSUPPORTED for the adaptive mode;
 *   DG_ERR_INVALID_ARG when a pending commit belongs to other caches, shapes
 *   or prefix array. */
dg_status dg_denoise_block_deferred(dg_ctx* ctx, const dg_sampler_cfg* cfg, int B,
                                    void* const* k_caches, void* const* v_caches, int Tmax,
                                    int32_t* prefix_len, int32_t* tokens_out,
                                    int32_t* steps_taken, void* stream);
/* dg_commit_pending: the commit forward of the context's pending block (its
 * K/V into slots [P_b - L, P_b); prefix_len is not changed, it was advanced
 * when the block ran).  DG_OK and nothing launched when none is pending;
 * DG_ERR_INVALID_ARG when the arguments are not the ones the pending block
 * ran with. */
dg_status dg_commit_pending(dg_ctx* ctx, int B, void* const* k_caches, void* const* v_caches,
                            int Tmax, const int32_t* prefix_len, void* stream);

/* dg_ar_decode: autoregressive decoding on the same model, the left-to-right
 * baseline the canvas is compared with ([JPH] "좌→우 순차 처리와의 대비"; [TR]
 * "수치").  n_steps single-token steps per row: a causal forward of the row's
 * current token at position P_b (its rotated K/V of every layer to cache slot
 * P_b), the final RMSNorm + LM head, then the greedy next token
 * argmax_v logits (ties to the lowest id; the pages fix no AR sampling rule);
 * P_b += 1.  The first step's input is tokens_in[b].
 *   tokens_in [B] i32 device; tokens_out [B, n_steps] i32 device (row-major);
 *   requires B <= max_batch and P_b + n_steps <= Tmax (the caller guarantees
 *   the latter).  Captured into one hipGraph per (B, n_steps, buffers) on a
 *   non-default stream when graphs are enabled. */
dg_status dg_ar_decode(dg_ctx* ctx, int B, int n_steps, const int32_t* tokens_in,
                       void* const* k_caches, void* const* v_caches, int Tmax,
                       int32_t* prefix_len, int32_t* tokens_out, void* stream);

/* dg_linear: the dense projections of a layer and the LM head ([TR]
 * "DiffusionGemma의 구성": a decoder whose layers project with dense matrices;
 * [GUIDE] "256토큰 Canvas 병렬 생성": the vocabulary logits of every canvas
 * position): out[m, n] = sum_k x[m, k] w[n, k], or out += that when
 * accumulate != 0.  The same kernels the decoder uses (QKV, O, router, LM
 * head).
 *   x [M, K] in dtype (DG_BF16 or DG_F32); w [N, K] in dtype and w_layout
 *   (DG_LAYOUT_TILED only with DG_BF16); out [M, N] in out_dtype: DG_BF16 or
 *   DG_F32 for bf16 inputs, DG_F32 for f32 inputs; accumulate needs DG_F32.
 *   bf16 inputs need N % 64 == 0 and K % 64 == 0; fp32 accumulation. */
dg_status dg_linear(const void* x, const void* w, void* out, int M, int N, int K, int dtype,
                    int w_layout, int out_dtype, int accumulate, void* stream);

/* ------------------------------------------------------------- utilities
 * Seeded synthetic data and checks used by tests and the benchmark. */

/* dst[i] = std * N(0,1) from Philox4x32-10 (counter (i / 4, 0, stream_id,
 * 0xFF000000), Box-Muller) in DG_F32 or DG_BF16. */
dg_status dg_fill_normal(void* dst, int dtype, size_t n, float std, uint64_t seed,
                         uint32_t stream_id, void* stream);
/* Per-row e4m3fn quantization of src [rows, cols] f32: scale = max|row| / 448,
 * q = round-to-nearest-even(src / scale) saturated to +-448. */
dg_status dg_quantize_fp8_rows(const float* src, uint8_t* q, float* scale, int64_t rows,
                               int cols, void* stream);
/* Repack weights [groups, N, K] from row-major into DG_LAYOUT_TILED (dst must
 * not alias src).  dtype: DG_BF16 or DG_FP8_E4M3 (any 1-byte type). */
dg_status dg_pack_weights(const void* src, void* dst, int64_t groups, int N, int K, int dtype,
                          void* stream);
/* OCP MXFP4 quantization of src [rows, cols] f32 (cols % 32 == 0; finite
 * values), row-major: codes [rows, cols / 2] (element 2j in the low nibble of
 * byte j), scales [rows, cols / 32] E8M0.  Per block of 32: shared exponent
 * floor(log2 amax) - 2 clamped to [-125, 127] (an all-zero block takes -125),
 * elements round to the nearest E2M1 value of v / 2^shared, ties to the even
 * mantissa, saturating at 6, sign kept (OCP Microscaling v1.0 conversion). */
dg_status dg_quantize_mxfp4(const float* src, uint8_t* codes, uint8_t* scales, int64_t rows,
                            int cols, void* stream);
/* Pack row-major MXFP4 codes [groups, N, K / 2] and scales [groups, N, K / 32]
 * into the tiled MXFP4 layout (dst: groups * N * K * 17 / 32 bytes, not
 * aliasing the inputs).  Needs N % 16 == 0 and K % 64 == 0. */
dg_status dg_pack_mxfp4(const uint8_t* codes, const uint8_t* scales, void* dst, int64_t groups,
                        int N, int K, void* stream);
/* Philox4x32-10 words for n counters: out[4i..4i+3] = Philox(ctr[4i..4i+3], seed). */
dg_status dg_philox(const uint32_t* counters, int64_t n, uint64_t seed, uint32_t* out,
                    void* stream);
/* The device Gumbel draw the sampler uses for each 32-bit word. */
dg_status dg_gumbel(const uint32_t* words, int64_t n, float* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DG_H_ */
