// C ABI: seeded device weights and fp8 quantization.
#include "kernels.h"

using namespace dg;

extern "C" {

dg_status dg_fill_normal(void* dst, int dtype, size_t n, float std, uint64_t seed,
                         uint32_t stream_id, void* stream) {
  set_error("");
  DG_CHECK_ARG(n == 0 || dst, "dg_fill_normal: null pointer");
  DG_CHECK_ARG(dtype == DG_F32 || dtype == DG_BF16, "dg_fill_normal: dtype must be f32 or bf16");
  DG_CHECK_SHAPE(n / 4 < (1ull << 62) / 256, "dg_fill_normal: n too large");
  return launch_fill_normal(dst, dtype, n, std, seed, stream_id, static_cast<hipStream_t>(stream));
}

dg_status dg_quantize_fp8_rows(const float* src, uint8_t* q, float* scale, int64_t rows, int cols,
                               void* stream) {
  set_error("");
  DG_CHECK_ARG(rows == 0 || (src && q && scale), "dg_quantize_fp8_rows: null pointer");
  DG_CHECK_SHAPE(rows >= 0 && rows < (1ll << 31) && cols > 0, "dg_quantize_fp8_rows: bad sizes");
  return launch_quantize_fp8_rows(src, q, scale, rows, cols, static_cast<hipStream_t>(stream));
}

dg_status dg_pack_weights(const void* src, void* dst, int64_t groups, int N, int K, int dtype,
                          void* stream) {
  set_error("");
  DG_CHECK_ARG(src && dst && src != dst, "dg_pack_weights: null or aliased pointer");
  DG_CHECK_ARG(dtype == DG_BF16 || dtype == DG_FP8_E4M3, "dg_pack_weights: dtype must be bf16 or fp8");
  DG_CHECK_SHAPE(groups > 0 && N > 0 && K > 0 && N % 16 == 0 && K % 64 == 0,
                 "dg_pack_weights: need N % 16 == 0 and K % 64 == 0");
  DG_CHECK_SHAPE(groups * N * static_cast<int64_t>(K) / 8 < (1ll << 31) * 256ll,
                 "dg_pack_weights: tensor too large");
  return launch_pack_weights(src, dst, groups, N, K, dtype == DG_BF16 ? 2 : 1,
                             static_cast<hipStream_t>(stream));
}

dg_status dg_quantize_mxfp4(const float* src, uint8_t* codes, uint8_t* scales, int64_t rows,
                            int cols, void* stream) {
  set_error("");
  DG_CHECK_ARG(rows == 0 || (src && codes && scales), "dg_quantize_mxfp4: null pointer");
  DG_CHECK_SHAPE(rows >= 0 && cols > 0 && cols % 32 == 0,
                 "dg_quantize_mxfp4: need rows >= 0 and cols % 32 == 0");
  DG_CHECK_SHAPE(rows * static_cast<int64_t>(cols) / 256 < (1ll << 31),
                 "dg_quantize_mxfp4: tensor too large");
  return launch_quantize_mxfp4(src, codes, scales, rows * static_cast<int64_t>(cols),
                               static_cast<hipStream_t>(stream));
}

dg_status dg_pack_mxfp4(const uint8_t* codes, const uint8_t* scales, void* dst, int64_t groups,
                        int N, int K, void* stream) {
  set_error("");
  DG_CHECK_ARG(codes && scales && dst && static_cast<const void*>(codes) != dst &&
                   static_cast<const void*>(scales) != dst,
               "dg_pack_mxfp4: null or aliased pointer");
  DG_CHECK_SHAPE(groups > 0 && N > 0 && K > 0 && N % 16 == 0 && K % 64 == 0,
                 "dg_pack_mxfp4: need N % 16 == 0 and K % 64 == 0");
  DG_CHECK_SHAPE(groups * N * static_cast<int64_t>(K) / 1024 < (1ll << 31),
                 "dg_pack_mxfp4: tensor too large");
  return launch_pack_mxfp4(codes, scales, dst, groups, N, K, static_cast<hipStream_t>(stream));
}

dg_status dg_linear(const void* x, const void* w, void* out, int M, int N, int K, int dtype,
                    int w_layout, int out_dtype, int accumulate, void* stream) {
  set_error("");
  DG_CHECK_ARG(x && w && out, "dg_linear: null pointer");
  DG_CHECK_ARG(dtype == DG_BF16 || dtype == DG_F32, "dg_linear: dtype must be DG_BF16 or DG_F32");
  DG_CHECK_ARG(w_layout == DG_LAYOUT_ROWMAJOR || (w_layout == DG_LAYOUT_TILED && dtype == DG_BF16),
               "dg_linear: bad w_layout (tiled needs bf16)");
  DG_CHECK_ARG(out_dtype == DG_F32 || (out_dtype == DG_BF16 && dtype == DG_BF16),
               "dg_linear: out_dtype must be DG_F32, or DG_BF16 with bf16 inputs");
  DG_CHECK_ARG(!accumulate || out_dtype == DG_F32, "dg_linear: accumulate needs an f32 output");
  DG_CHECK_SHAPE(M > 0 && N > 0 && K > 0, "dg_linear: sizes must be positive");
  if (dtype == DG_BF16)
    DG_CHECK_SHAPE(N % 64 == 0 && K % 64 == 0, "dg_linear: bf16 needs N % 64 == 0 and K % 64 == 0");
  return launch_gemm(x, w, out, M, N, K, dtype, w_layout, out_dtype,
                     accumulate ? kAccumulateF32 : kStore, static_cast<hipStream_t>(stream));
}

}  // extern "C"
