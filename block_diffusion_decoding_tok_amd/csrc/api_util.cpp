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

}  // extern "C"
