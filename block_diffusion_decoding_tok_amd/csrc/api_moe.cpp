// C ABI: MoE routing and expert FFN.
#include "kernels.h"

using namespace dg;

extern "C" {

size_t dg_moe_route_workspace_size(int T, int E, int k) {
  if (T <= 0 || E <= 0 || k <= 0) return 0;
  return moe_route_workspace_bytes(T, E, k);
}

dg_status dg_moe_route(const float* router_logits, int T, int E, int k, int32_t* topk_ids,
                       float* gates, int32_t* expert_offsets, int32_t* sorted_rows, void* ws,
                       size_t ws_bytes, void* stream) {
  set_error("");
  DG_CHECK_ARG(router_logits && topk_ids && gates && expert_offsets && sorted_rows,
               "dg_moe_route: null pointer");
  DG_CHECK_SHAPE(T > 0 && E > 0 && E <= 256, "dg_moe_route: need T > 0 and 0 < E <= 256");
  DG_CHECK_SHAPE(k > 0 && k <= E && k <= 16, "dg_moe_route: need 0 < k <= min(E, 16)");
  DG_CHECK_SHAPE(static_cast<int64_t>(T) * k < (1ll << 31), "dg_moe_route: T * k too large");
  if (ws_bytes < moe_route_workspace_bytes(T, E, k))
    return fail(DG_ERR_WORKSPACE, "dg_moe_route: workspace too small");
  return launch_moe_route(router_logits, T, E, k, topk_ids, gates, expert_offsets, sorted_rows,
                          ws, static_cast<hipStream_t>(stream));
}

size_t dg_moe_ffn_workspace_size(int T, int D, int I, int E, int k, int x_dtype) {
  if (T <= 0 || D <= 0 || I <= 0 || E <= 0 || k <= 0) return 0;
  return moe_ffn_workspace_bytes(T, D, I, E, k, x_dtype);
}

dg_status dg_moe_ffn(const void* x, int x_dtype, const void* w_gate_up, const void* w_down,
                     int w_dtype, int w_layout, const float* s_gate_up, const float* s_down,
                     const int32_t* topk_ids, const float* gates, const int32_t* expert_offsets,
                     const int32_t* sorted_rows, int T, int D, int I, int E, int k, float* y,
                     void* ws, size_t ws_bytes, void* stream) {
  set_error("");
  DG_CHECK_ARG(x && w_gate_up && w_down && topk_ids && gates && expert_offsets && sorted_rows && y,
               "dg_moe_ffn: null pointer");
  DG_CHECK_ARG(x_dtype == DG_BF16 || x_dtype == DG_F32, "dg_moe_ffn: x_dtype must be DG_BF16 or DG_F32");
  DG_CHECK_ARG(w_dtype == DG_BF16 || w_dtype == DG_F32 || w_dtype == DG_FP8_E4M3,
               "dg_moe_ffn: bad w_dtype");
  DG_CHECK_ARG((x_dtype == DG_F32) == (w_dtype == DG_F32),
               "dg_moe_ffn: f32 activations go with f32 weights only");
  DG_CHECK_ARG(w_layout == DG_LAYOUT_ROWMAJOR || w_layout == DG_LAYOUT_TILED,
               "dg_moe_ffn: bad w_layout");
  DG_CHECK_ARG(w_layout == DG_LAYOUT_ROWMAJOR || x_dtype != DG_F32,
               "dg_moe_ffn: the tiled layout needs bf16 activations");
  DG_CHECK_ARG(w_dtype != DG_FP8_E4M3 || (s_gate_up && s_down),
               "dg_moe_ffn: fp8 weights need s_gate_up and s_down");
  DG_CHECK_SHAPE(T > 0 && E > 0 && E <= 256 && k > 0 && k <= E && k <= 16,
                 "dg_moe_ffn: bad T / E / k");
  DG_CHECK_SHAPE(D > 0 && I > 0 && D % 4 == 0, "dg_moe_ffn: bad D / I");
  if (x_dtype != DG_F32)
    DG_CHECK_SHAPE(D % 128 == 0 && I % 64 == 0,
                   "dg_moe_ffn: the MFMA path needs D % 128 == 0 and I % 64 == 0");
  if (ws == nullptr || ws_bytes < moe_ffn_workspace_bytes(T, D, I, E, k, x_dtype))
    return fail(DG_ERR_WORKSPACE, "dg_moe_ffn: workspace too small");
  return launch_moe_ffn(x, x_dtype, w_gate_up, w_down, w_dtype, w_layout, s_gate_up, s_down,
                        topk_ids, gates,
                        expert_offsets, sorted_rows, T, D, I, E, k, y, ws,
                        static_cast<hipStream_t>(stream));
}

}  // extern "C"
