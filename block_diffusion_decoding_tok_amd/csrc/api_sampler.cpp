// C ABI: sampler step, canvas init, Philox and Gumbel test hooks.
#include <cmath>

#include "kernels.h"

using namespace dg;

extern "C" {

size_t dg_sampler_workspace_size(int B, int L, int V) {
  if (B <= 0 || L <= 0 || V <= 0) return 0;
  return sampler_workspace_bytes(B, L, V);
}

}  // extern "C"

namespace dg {
// Host checks of one sampler step (everything but the workspace).
dg_status check_sampler_step(const void* logits, int logit_dtype, int B, int L, int V, int step,
                             const dg_sampler_cfg* cfg, const int32_t* prefix_len,
                             const int32_t* tokens, const uint8_t* committed,
                             const uint8_t* renoised, const float* maxprob,
                             const float* entropy, const float* mean_entropy,
                             const int32_t* done) {
  DG_CHECK_ARG(cfg != nullptr, "dg_sampler_step: cfg is null");
  DG_CHECK_ARG(logits && prefix_len && tokens && committed && renoised && maxprob && entropy &&
                   mean_entropy && done,
               "dg_sampler_step: null tensor pointer");
  DG_CHECK_ARG(logit_dtype == DG_BF16 || logit_dtype == DG_F32,
               "dg_sampler_step: logit_dtype must be DG_BF16 or DG_F32");
  DG_CHECK_SHAPE(B > 0 && B < (1 << 24), "dg_sampler_step: B must be in [1, 2^24)");
  DG_CHECK_SHAPE(L > 0 && L <= 4096, "dg_sampler_step: L must be in [1, 4096]");
  DG_CHECK_SHAPE(V > 0 && V % 8 == 0, "dg_sampler_step: V must be a positive multiple of 8");
  DG_CHECK_SHAPE(cfg->max_steps >= 1, "dg_sampler_step: max_steps must be >= 1");
  DG_CHECK_SHAPE(cfg->fixed_steps >= 0 && cfg->fixed_steps <= cfg->max_steps,
                 "dg_sampler_step: fixed_steps must be in [0, max_steps]");
  const int limit = cfg->fixed_steps > 0 ? cfg->fixed_steps : cfg->max_steps;
  DG_CHECK_SHAPE(step >= 0 && step < limit, "dg_sampler_step: step outside the schedule");
  DG_CHECK_ARG(cfg->temp_start > 0.f && cfg->temp_end > 0.f,
               "dg_sampler_step: temperatures must be positive");
  DG_CHECK_ARG(cfg->commit_policy == DG_COMMIT_MAXPROB ||
                   (cfg->commit_policy == DG_COMMIT_ENTROPY_BOUND && cfg->entropy_bound >= 0.f &&
                    cfg->entropy_bound < INFINITY),
               "dg_sampler_step: bad commit_policy / entropy_bound");
  return DG_OK;
}
}  // namespace dg

extern "C" {

dg_status dg_sampler_step(const void* logits, int logit_dtype, int B, int L, int V, int step,
                          const dg_sampler_cfg* cfg, const int32_t* prefix_len, int32_t* tokens,
                          uint8_t* committed, uint8_t* renoised, float* maxprob, float* entropy,
                          float* mean_entropy, int32_t* done, int32_t* status, void* ws,
                          size_t ws_bytes, void* stream) {
  set_error("");
  const dg_status st = check_sampler_step(logits, logit_dtype, B, L, V, step, cfg, prefix_len,
                                          tokens, committed, renoised, maxprob, entropy,
                                          mean_entropy, done);
  if (st != DG_OK) return st;
  if (ws_bytes < sampler_workspace_bytes(B, L, V) || ws == nullptr)
    return fail(DG_ERR_WORKSPACE, "dg_sampler_step: workspace too small");
  return launch_sampler(logits, logit_dtype, B, L, V, step, *cfg, prefix_len, tokens, committed,
                        renoised, maxprob, entropy, mean_entropy, done, status, nullptr, ws,
                        static_cast<hipStream_t>(stream));
}

dg_status dg_init_canvas(const int32_t* prefix_len, int B, int L, int V, uint64_t seed,
                         int32_t* tokens, uint8_t* committed, int32_t* done, void* stream) {
  set_error("");
  DG_CHECK_ARG(prefix_len && tokens && committed && done, "dg_init_canvas: null pointer");
  DG_CHECK_SHAPE(B > 0 && B < (1 << 24) && L > 0 && V > 0, "dg_init_canvas: bad sizes");
  DG_CHECK_SHAPE(static_cast<int64_t>(B) * L < (1ll << 31), "dg_init_canvas: B * L too large");
  return launch_init_canvas(prefix_len, B, L, V, seed, tokens, committed, done,
                            static_cast<hipStream_t>(stream));
}

dg_status dg_philox(const uint32_t* counters, int64_t n, uint64_t seed, uint32_t* out,
                    void* stream) {
  set_error("");
  DG_CHECK_ARG(n >= 0, "dg_philox: n < 0");
  DG_CHECK_ARG(n == 0 || (counters && out), "dg_philox: null pointer");
  return launch_philox(counters, n, seed, out, static_cast<hipStream_t>(stream));
}

dg_status dg_gumbel(const uint32_t* words, int64_t n, float* out, void* stream) {
  set_error("");
  DG_CHECK_ARG(n >= 0, "dg_gumbel: n < 0");
  DG_CHECK_ARG(n == 0 || (words && out), "dg_gumbel: null pointer");
  return launch_gumbel(words, n, out, static_cast<hipStream_t>(stream));
}

}  // extern "C"
