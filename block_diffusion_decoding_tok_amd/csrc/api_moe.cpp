// C ABI: MoE routing and expert FFN.
#include <cstdio>

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

}  // extern "C"

// Argument checks shared by the expert FFN entry points.
static dg_status check_ffn(const char* fn, int x_dtype, int w_dtype, int w_layout,
                           const float* scales_a, const float* scales_b, int T, int D, int I,
                           int E, int k) {
  char msg[160];
  auto bad = [&](dg_status code, const char* what) {
    snprintf(msg, sizeof(msg), "%s: %s", fn, what);
    return fail(code, msg);
  };
  if (!(x_dtype == DG_BF16 || x_dtype == DG_F32))
    return bad(DG_ERR_INVALID_ARG, "activation dtype must be DG_BF16 or DG_F32");
  if (!(w_dtype == DG_BF16 || w_dtype == DG_F32 || w_dtype == DG_FP8_E4M3 || w_dtype == DG_MXFP4))
    return bad(DG_ERR_INVALID_ARG, "bad w_dtype");
  if (w_dtype == DG_MXFP4 && w_layout != DG_LAYOUT_TILED)
    return bad(DG_ERR_INVALID_ARG, "MXFP4 weights must be tile-packed (DG_LAYOUT_TILED)");
  if ((x_dtype == DG_F32) != (w_dtype == DG_F32))
    return bad(DG_ERR_INVALID_ARG, "f32 activations go with f32 weights only");
  if (!(w_layout == DG_LAYOUT_ROWMAJOR || w_layout == DG_LAYOUT_TILED))
    return bad(DG_ERR_INVALID_ARG, "bad w_layout");
  if (w_layout == DG_LAYOUT_TILED && x_dtype == DG_F32)
    return bad(DG_ERR_INVALID_ARG, "the tiled layout needs bf16 activations");
  if (w_dtype == DG_FP8_E4M3 && !(scales_a && scales_b))
    return bad(DG_ERR_INVALID_ARG, "fp8 weights need their per-row scales");
  if (!(T > 0 && E > 0 && E <= 256 && k > 0 && k <= E && k <= 16))
    return bad(DG_ERR_SHAPE, "bad T / E / k");
  if (static_cast<int64_t>(T) * k >= (1ll << 31)) return bad(DG_ERR_SHAPE, "T * k too large");
  if (!(D > 0 && I > 0 && D % 4 == 0)) return bad(DG_ERR_SHAPE, "bad D / I");
  if (x_dtype != DG_F32 && !(D % 128 == 0 && I % 64 == 0))
    return bad(DG_ERR_SHAPE, "the MFMA path needs D % 128 == 0 and I % 64 == 0");
  return DG_OK;
}

extern "C" {

dg_status dg_moe_ffn(const void* x, int x_dtype, const void* w_gate_up, const void* w_down,
                     int w_dtype, int w_layout, const float* s_gate_up, const float* s_down,
                     const int32_t* topk_ids, const float* gates, const int32_t* expert_offsets,
                     const int32_t* sorted_rows, int T, int D, int I, int E, int k, float* y,
                     void* ws, size_t ws_bytes, void* stream) {
  set_error("");
  DG_CHECK_ARG(x && w_gate_up && w_down && topk_ids && gates && expert_offsets && sorted_rows && y,
               "dg_moe_ffn: null pointer");
  const dg_status st = check_ffn("dg_moe_ffn", x_dtype, w_dtype, w_layout, s_gate_up, s_down, T,
                                 D, I, E, k);
  if (st != DG_OK) return st;
  if (ws == nullptr || ws_bytes < moe_ffn_workspace_bytes(T, D, I, E, k, x_dtype))
    return fail(DG_ERR_WORKSPACE, "dg_moe_ffn: workspace too small");
  return launch_moe_ffn(x, x_dtype, w_gate_up, w_down, w_dtype, w_layout, s_gate_up, s_down,
                        topk_ids, gates, expert_offsets, sorted_rows, T, D, I, E, k, y, ws,
                        static_cast<hipStream_t>(stream));
}

dg_status dg_moe_gate_up(const void* x, int x_dtype, const void* w_gate_up, int w_dtype,
                         int w_layout, const float* s_gate_up, const int32_t* expert_offsets,
                         const int32_t* sorted_rows, int T, int D, int I, int E, int k, void* h,
                         void* stream) {
  set_error("");
  DG_CHECK_ARG(x && w_gate_up && expert_offsets && sorted_rows && h,
               "dg_moe_gate_up: null pointer");
  const dg_status st = check_ffn("dg_moe_gate_up", x_dtype, w_dtype, w_layout, s_gate_up,
                                 s_gate_up, T, D, I, E, k);
  if (st != DG_OK) return st;
  return launch_moe_gate_up(x, x_dtype, w_gate_up, w_dtype, w_layout, s_gate_up, expert_offsets,
                            sorted_rows, T, D, I, E, k, h, static_cast<hipStream_t>(stream));
}

dg_status dg_moe_down(const void* h, int h_dtype, const void* w_down, int w_dtype, int w_layout,
                      const float* s_down, const float* gates, const int32_t* expert_offsets,
                      const int32_t* sorted_rows, int T, int D, int I, int E, int k, void* y_slot,
                      void* stream) {
  set_error("");
  DG_CHECK_ARG(h && w_down && gates && expert_offsets && sorted_rows && y_slot,
               "dg_moe_down: null pointer");
  const dg_status st = check_ffn("dg_moe_down", h_dtype, w_dtype, w_layout, s_down, s_down, T, D,
                                 I, E, k);
  if (st != DG_OK) return st;
  return launch_moe_down(h, h_dtype, w_down, w_dtype, w_layout, s_down, gates, expert_offsets,
                         sorted_rows, T, D, I, E, k, y_slot, static_cast<hipStream_t>(stream));
}

dg_status dg_moe_combine(const void* y_slot, int dtype, int T, int D, int k, float* y,
                         void* stream) {
  set_error("");
  DG_CHECK_ARG(y_slot && y, "dg_moe_combine: null pointer");
  DG_CHECK_ARG(dtype == DG_BF16 || dtype == DG_F32, "dg_moe_combine: dtype must be DG_BF16 or DG_F32");
  DG_CHECK_SHAPE(T > 0 && D > 0 && D % 4 == 0 && k > 0 && k <= 16,
                 "dg_moe_combine: need T > 0, D % 4 == 0, 0 < k <= 16");
  DG_CHECK_SHAPE(static_cast<int64_t>(T) * k * D < (1ll << 40), "dg_moe_combine: too large");
  return launch_moe_combine(y_slot, dtype, T, D, k, y, static_cast<hipStream_t>(stream));
}

}  // extern "C"
