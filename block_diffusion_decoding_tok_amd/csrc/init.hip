// Seeded synthetic weights on the device (the benchmark's 27 GB model is
// generated here rather than on the host) and per-row fp8 quantization.
//   fill_normal: Philox4x32-10 counter (i / 4 lo, i / 4 hi, stream_id,
//   0xFF000000) -> four 24-bit uniforms -> two Box-Muller pairs.
//   quantize: scale = max|row| / 448; byte = e4m3fn round-to-nearest-even of
//   x / scale, saturated to +-448.
//   pack: row-major weights -> DG_LAYOUT_TILED.
#include "common.h"
#include "kernels.h"
#include "philox.h"

namespace dg {

template <typename T>
__global__ void fill_normal_kernel(T* __restrict__ dst, size_t n, float std, uint32_t k0,
                                   uint32_t k1, uint32_t stream_id) {
  const size_t q = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;   // quad index
  const size_t i0 = q * 4;
  if (i0 >= n) return;
  const Philox4 r = philox4x32_10(static_cast<uint32_t>(q), static_cast<uint32_t>(q >> 32),
                                  stream_id, 0xFF000000u, k0, k1);
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
  float z[4];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const float u1 = (static_cast<float>(w[2 * p] >> 8) + 0.5f) * 0x1.0p-24f;
    const float u2 = (static_cast<float>(w[2 * p + 1] >> 8) + 0.5f) * 0x1.0p-24f;
    const float rad = sqrtf(-2.0f * logf(u1));
    float s, c;
    sincosf(6.283185307179586f * u2, &s, &c);
    z[2 * p] = rad * c;
    z[2 * p + 1] = rad * s;
  }
  for (int j = 0; j < 4 && i0 + j < n; ++j) Elem<T>::store(dst, i0 + j, z[j] * std);
}

__device__ __forceinline__ uint8_t f32_to_e4m3fn_rne(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 31) << 7;
  float a = fminf(fabsf(v), 448.0f);
  int E = static_cast<int>((__float_as_uint(a) >> 23) & 0xFF) - 127;
  uint32_t bits;
  if (a == 0.0f) {
    bits = 0;
  } else if (E < -6) {                         // subnormal: multiples of 2^-9
    bits = static_cast<uint32_t>(rintf(a * 512.0f));   // 8 rounds up into the normal range
  } else {
    float q = rintf(ldexpf(a, 3 - E));         // in [8, 16]
    if (q >= 16.0f) { q = 8.0f; ++E; }
    bits = (static_cast<uint32_t>(E + 7) << 3) | (static_cast<uint32_t>(q) - 8u);
  }
  return static_cast<uint8_t>(sign | bits);
}

__global__ __launch_bounds__(256) void quantize_rows_kernel(const float* __restrict__ src,
                                                            uint8_t* __restrict__ q,
                                                            float* __restrict__ scale, int cols) {
  const int64_t row = blockIdx.x;
  const float* s = src + row * cols;
  float m = 0.f;
  for (int c = threadIdx.x; c < cols; c += blockDim.x) m = fmaxf(m, fabsf(s[c]));
  m = warp_max(m);
  __shared__ float s_m[4];
  if ((threadIdx.x & 63) == 0) s_m[threadIdx.x >> 6] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
  const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
  if (threadIdx.x == 0) scale[row] = sc;
  for (int c = threadIdx.x; c < cols; c += blockDim.x) q[row * cols + c] = f32_to_e4m3fn_rne(s[c] / sc);
}

// Row-major [G, N, K] -> tile-packed (16 rows x 64 k blocks in wave-load
// order); one thread per 16-byte piece of the destination.
__global__ void pack_weights_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                    int64_t pieces, int N, int K, int elem_bytes) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (q >= pieces) return;
  const int per_block = 1024 * elem_bytes / 16;        // 64 (1-byte) or 128 (2-byte) pieces
  const int64_t blk = q / per_block;
  const int within = static_cast<int>(q % per_block);
  const int lane = within % 64, h = within / 64;
  const int r = lane % 16, g4 = lane / 16;
  const int64_t NC = K / 64, NT = N / 16;
  const int64_t c = blk % NC;
  const int64_t gt = blk / NC;                          // g * NT + t
  const int64_t g = gt / NT, t = gt % NT;
  const int vals = 16 / elem_bytes;                     // values per piece
  const int64_t elem = (g * N + 16 * t + r) * static_cast<int64_t>(K) + 64 * c + 16 * g4 + vals * h;
  dst[q] = src[elem * elem_bytes / 16];
}

dg_status launch_pack_weights(const void* src, void* dst, int64_t groups, int N, int K,
                              int elem_bytes, hipStream_t stream) {
  const int64_t pieces = groups * N * static_cast<int64_t>(K) * elem_bytes / 16;
  if (pieces == 0) return DG_OK;
  pack_weights_kernel<<<static_cast<unsigned>((pieces + 255) / 256), 256, 0, stream>>>(
      static_cast<const uint4*>(src), static_cast<uint4*>(dst), pieces, N, K, elem_bytes);
  DG_LAUNCH_CHECK();
  return DG_OK;
}

dg_status launch_fill_normal(void* dst, int dtype, size_t n, float std, uint64_t seed,
                             uint32_t stream_id, hipStream_t stream) {
  if (n == 0) return DG_OK;
  const size_t quads = (n + 3) / 4;
  const unsigned blocks = static_cast<unsigned>((quads + 255) / 256);
  const uint32_t k0 = static_cast<uint32_t>(seed), k1 = static_cast<uint32_t>(seed >> 32);
  if (dtype == DG_BF16)
    fill_normal_kernel<bf16_t><<<blocks, 256, 0, stream>>>(static_cast<bf16_t*>(dst), n, std, k0, k1, stream_id);
  else
    fill_normal_kernel<float><<<blocks, 256, 0, stream>>>(static_cast<float*>(dst), n, std, k0, k1, stream_id);
  DG_LAUNCH_CHECK();
  return DG_OK;
}

dg_status launch_quantize_fp8_rows(const float* src, uint8_t* q, float* scale, int64_t rows,
                                   int cols, hipStream_t stream) {
  if (rows == 0) return DG_OK;
  quantize_rows_kernel<<<static_cast<unsigned>(rows), 256, 0, stream>>>(src, q, scale, cols);
  DG_LAUNCH_CHECK();
  return DG_OK;
}

}  // namespace dg
