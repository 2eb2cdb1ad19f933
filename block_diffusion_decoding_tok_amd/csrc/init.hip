// Seeded synthetic weights on the device (the benchmark's 27 GB model is
// generated here rather than on the host) and per-row fp8 quantization.
//   fill_normal: Philox4x32-10 counter (i / 4 lo, i / 4 hi, stream_id,
//   0xFF000000) -> four 24-bit uniforms -> two Box-Muller pairs.
//   quantize: scale = max|row| / 448; byte = e4m3fn round-to-nearest-even of
//   x / scale, saturated to +-448.
//   pack: row-major weights -> DG_LAYOUT_TILED.
//   MXFP4: OCP block quantization (32 k per E8M0 scale) and its tiled pack.
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
// order; one matrix: a tile's blocks contiguous, block (t, c) at t K/64 + c; a
// stack of G > 1: block (g, t, c) at (c G + g) N/16 + t, every expert's k
// chunk c together); one thread per 16-byte piece of the destination.
__global__ void pack_weights_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                    int64_t pieces, int64_t G, int N, int K, int elem_bytes) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (q >= pieces) return;
  const int per_block = 1024 * elem_bytes / 16;        // 64 (1-byte) or 128 (2-byte) pieces
  const int64_t blk = q / per_block;
  const int within = static_cast<int>(q % per_block);
  const int lane = within % 64, h = within / 64;
  const int r = lane % 16, g4 = lane / 16;
  const int64_t NC = K / 64, NT = N / 16;
  int64_t g, t, c;
  if (G == 1) {
    g = 0; t = blk / NC; c = blk % NC;
  } else {
    t = blk % NT;
    const int64_t cg = blk / NT;                        // c * G + g
    g = cg % G; c = cg / G;
  }
  const int vals = 16 / elem_bytes;                     // values per piece
  const int64_t elem = (g * N + 16 * t + r) * static_cast<int64_t>(K) + 64 * c + 16 * g4 + vals * h;
  dst[q] = src[elem * elem_bytes / 16];
}

dg_status launch_pack_weights(const void* src, void* dst, int64_t groups, int N, int K,
                              int elem_bytes, hipStream_t stream) {
  const int64_t pieces = groups * N * static_cast<int64_t>(K) * elem_bytes / 16;
  if (pieces == 0) return DG_OK;
  pack_weights_kernel<<<static_cast<unsigned>((pieces + 255) / 256), 256, 0, stream>>>(
      static_cast<const uint4*>(src), static_cast<uint4*>(dst), pieces, groups, N, K, elem_bytes);
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

// ------------------------------------------------------------------ MXFP4
// One lane per element, 32 consecutive lanes per block: the block's amax by a
// max over the magnitudes' bit patterns (ordered like the values for
// non-negative floats), shared exponent floor(log2 amax) - 2 from amax's
// exponent field (a zero or subnormal amax falls to the clamp), then the
// element's E2M1 magnitude by counting the grid midpoints it passes: at a
// midpoint the comparison is strict where the lower neighbour has the even
// mantissa and inclusive where the upper one does (round half to even);
// beyond 5 everything saturates to 6.  v * 2^-shared is exact (a power of two
// within the normal range), so the decisions are exact.
__global__ __launch_bounds__(256) void quantize_mxfp4_kernel(const float* __restrict__ src,
                                                             uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales,
                                                             int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const bool ok = i < n;                      // n % 32 == 0: a block is all in or all out
  const float v = src[ok ? i : 0];
  uint32_t m = __float_as_uint(v) & 0x7fffffffu;
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), o)));
  const int shared = min(max(static_cast<int>(m >> 23) - 127 - 2, -125), 127);
  const float a = fabsf(v) * __uint_as_float(static_cast<uint32_t>(127 - shared) << 23);
  const uint32_t mag = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
                       (a >= 3.5f) + (a > 5.0f);
  const uint32_t code = mag | ((__float_as_uint(v) >> 31) << 3);
  const uint32_t hi = static_cast<uint32_t>(__shfl_down(static_cast<int>(code), 1));
  if (ok && (threadIdx.x & 1) == 0) codes[i / 2] = static_cast<uint8_t>(code | (hi << 4));
  if (ok && (threadIdx.x & 31) == 0) scales[i / 32] = static_cast<uint8_t>(shared + 127);
}

dg_status launch_quantize_mxfp4(const float* src, uint8_t* codes, uint8_t* scales, int64_t n,
                                hipStream_t stream) {
  if (n == 0) return DG_OK;
  quantize_mxfp4_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, stream>>>(src, codes,
                                                                                   scales, n);
  DG_LAUNCH_CHECK();
  return DG_OK;
}

// Row-major codes [G, N, K / 2] + scales [G, N, K / 32] -> tiled MXFP4 blocks
// of 544 bytes (16 rows x 64 k); one thread per 8-byte word of the
// destination: words 0..63 are lane r + 16 q's codes (row r, k 16 q ..
// 16 q + 15), words 64..67 the 32 scale bytes (16 h + r: row r, half h).
__global__ void pack_mxfp4_kernel(const uint8_t* __restrict__ codes,
                                  const uint8_t* __restrict__ scales, uint2* __restrict__ dst,
                                  int64_t words, int N, int K) {
  const int64_t w = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (w >= words) return;
  const int64_t blk = w / 68;
  const int within = static_cast<int>(w % 68);
  const int64_t NC = K / 64, NT = N / 16;
  const int64_t c = blk % NC;
  const int64_t gt = blk / NC;                          // g * NT + t
  const int64_t g = gt / NT, t = gt % NT;
  const int64_t row0 = g * N + 16 * t;                  // first row of the tile
  if (within < 64) {
    const int r = within % 16, q = within / 16;
    dst[w] = *reinterpret_cast<const uint2*>(codes + (row0 + r) * (K / 2) + 32 * c + 8 * q);
  } else {
    uint32_t b[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int byte = 8 * (within - 64) + j, h = byte / 16, r = byte % 16;
      b[j] = scales[(row0 + r) * (K / 32) + 2 * c + h];
    }
    dst[w] = make_uint2(b[0] | b[1] << 8 | b[2] << 16 | b[3] << 24,
                        b[4] | b[5] << 8 | b[6] << 16 | b[7] << 24);
  }
}

dg_status launch_pack_mxfp4(const uint8_t* codes, const uint8_t* scales, void* dst,
                            int64_t groups, int N, int K, hipStream_t stream) {
  const int64_t words = groups * (N / 16) * static_cast<int64_t>(K / 64) * 68;
  if (words == 0) return DG_OK;
  pack_mxfp4_kernel<<<static_cast<unsigned>((words + 255) / 256), 256, 0, stream>>>(
      codes, scales, static_cast<uint2*>(dst), words, N, K);
  DG_LAUNCH_CHECK();
  return DG_OK;
}

}  // namespace dg
