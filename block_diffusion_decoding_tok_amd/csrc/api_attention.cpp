// C ABI: canvas attention and KV commit.
#include "kernels.h"

using namespace dg;

static dg_status check_attn_shapes(const char* fn, int B, int L, int Hq, int Hkv, int dh,
                                   int Tmax, int dtype) {
  DG_CHECK_ARG(dtype == DG_BF16 || dtype == DG_F32, std::string(fn) + ": dtype must be DG_BF16 or DG_F32");
  DG_CHECK_SHAPE(B > 0 && L > 0 && Hq > 0 && Hkv > 0 && Tmax > 0, std::string(fn) + ": sizes must be positive");
  DG_CHECK_SHAPE(Hq % Hkv == 0, std::string(fn) + ": Hq must be a multiple of Hkv");
  DG_CHECK_SHAPE(L <= Tmax, std::string(fn) + ": block longer than the cache");
  if (dtype == DG_BF16)
    DG_CHECK_SHAPE(dh == 128, std::string(fn) + ": the bf16 path needs head_dim 128");
  else
    DG_CHECK_SHAPE(dh >= 2 && dh <= 128 && dh % 2 == 0, std::string(fn) + ": f32 head_dim must be even and <= 128");
  DG_CHECK_SHAPE(static_cast<int64_t>(B) * Hkv * Tmax * dh < (1ll << 40), std::string(fn) + ": cache too large");
  return DG_OK;
}

extern "C" {

size_t dg_attention_workspace_size(int B, int Lq, int Hq, int Hkv, int dh, int Tmax, int dtype) {
  if (B <= 0 || Lq <= 0 || Hq <= 0 || Hkv <= 0 || dh <= 0 || Tmax <= 0 || Hq % Hkv) return 0;
  return attention_workspace_bytes(B, Lq, Hq, Hkv, dh, Tmax, dtype);
}

dg_status dg_canvas_attention(const void* q, const void* k_new, const void* v_new, void* k_cache,
                              void* v_cache, const int32_t* prefix_len, int B, int Lq, int Hq,
                              int Hkv, int dh, int Tmax, int mask_mode, float rope_theta,
                              int dtype, void* out, void* ws, size_t ws_bytes, void* stream) {
  set_error("");
  DG_CHECK_ARG(q && k_new && v_new && k_cache && v_cache && prefix_len && out,
               "dg_canvas_attention: null pointer");
  DG_CHECK_ARG(mask_mode == DG_MASK_CANVAS || mask_mode == DG_MASK_CAUSAL,
               "dg_canvas_attention: bad mask_mode");
  DG_CHECK_ARG(rope_theta > 1.f, "dg_canvas_attention: rope_theta must be > 1");
  dg_status st = check_attn_shapes("dg_canvas_attention", B, Lq, Hq, Hkv, dh, Tmax, dtype);
  if (st != DG_OK) return st;
  if (ws == nullptr || ws_bytes < attention_workspace_bytes(B, Lq, Hq, Hkv, dh, Tmax, dtype))
    return fail(DG_ERR_WORKSPACE, "dg_canvas_attention: workspace too small");
  AttnArgs a{q, k_new, v_new, static_cast<int64_t>(Hq) * dh, static_cast<int64_t>(Hkv) * dh,
             k_cache, v_cache, prefix_len, B, Lq, Hq, Hkv, dh, Tmax, mask_mode, rope_theta,
             dtype, out};
  return launch_attention(a, ws, static_cast<hipStream_t>(stream));
}

dg_status dg_commit_block(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                          int32_t* prefix_len, int B, int L, int Hkv, int dh, int Tmax,
                          float rope_theta, int dtype, void* stream) {
  set_error("");
  DG_CHECK_ARG(k_new && v_new && k_cache && v_cache && prefix_len, "dg_commit_block: null pointer");
  DG_CHECK_ARG(rope_theta > 1.f, "dg_commit_block: rope_theta must be > 1");
  dg_status st = check_attn_shapes("dg_commit_block", B, L, Hkv, Hkv, dh, Tmax, dtype);
  if (st != DG_OK) return st;
  return launch_commit(k_new, v_new, static_cast<int64_t>(Hkv) * dh, k_cache, v_cache,
                       prefix_len, B, L, Hkv, dh, Tmax, rope_theta, dtype, true,
                       static_cast<hipStream_t>(stream));
}

}  // extern "C"
