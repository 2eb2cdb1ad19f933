// Dense projections (QKV, O, router, LM head), RMSNorm and the embedding
// gather of the decoder layer.
//
//   bf16: gemm_stream_kernel (gemm_mfma.h) in dense mode -- 64 weight rows x
//         64 tokens per workgroup (16 tokens for narrow outputs), the token
//         tiles of the same rows adjacent so they share one XCD's L2.
//   f32:  plain SIMT kernels (parity path of the tiny fp32 model).
// RMSNorm: x / sqrt(mean(x^2) + 1e-6), unit gain, f32 statistics.
#include "common.h"
#include "gemm_mfma.h"
#include "kernels.h"

namespace dg {

// projection-sized outputs (QKV, O, router): split-K register streaming
constexpr int kSplitNR = 2;
// other shapes: 64 rows x 64 tokens per workgroup, LDS-staged tokens
constexpr int kDenseRT = 1, kDenseTB = 4, kDenseKS = 2, kDensePF = 2;
// up to 256 tokens: register streaming, 16 tokens per tile, ring of 4 chunks
constexpr int kDenseNR = 4;
// vocabulary-sized outputs (LM head): 128 rows x 256 tokens, so each weight
// row is read once per 256 tokens
constexpr int kWideRT = 2, kWideTB = 16, kWideKS = 1, kWidePF = 2;

__global__ void gemm_f32_kernel(const float* __restrict__ A, const float* __restrict__ W,
                                float* __restrict__ C, int M, int N, int K, int accumulate) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  const int m = blockIdx.y;
  if (n >= N) return;
  const float* a = A + static_cast<int64_t>(m) * K;
  const float* w = W + static_cast<int64_t>(n) * K;
  float acc = 0.f;
  for (int k = 0; k < K; ++k) acc = fmaf(a[k], w[k], acc);
  float* c = C + static_cast<int64_t>(m) * N + n;
  *c = accumulate ? *c + acc : acc;
}

template <bool TILED>
static void launch_gemm_bf16(GemmArgs& g, int M, int N, int K, hipStream_t stream);

dg_status launch_gemm(const void* A, const void* W, void* C, int M, int N, int K, int dtype,
                      int w_layout, int out_dtype, GemmEpilogue ep, hipStream_t stream) {
  if (dtype == DG_F32) {
    dim3 grid((N + 127) / 128, M);
    gemm_f32_kernel<<<grid, 128, 0, stream>>>(static_cast<const float*>(A),
                                              static_cast<const float*>(W),
                                              static_cast<float*>(C), M, N, K,
                                              ep == kAccumulateF32);
    DG_LAUNCH_CHECK();
    return DG_OK;
  }
  GemmArgs g{};
  g.W = W; g.X = static_cast<const bf16_t*>(A);
  g.N = N; g.K = K; g.M = M; g.n_groups = 1;
  g.out = C;
  g.out_dtype = ep == kAccumulateF32 ? DG_F32 : out_dtype;
  g.accumulate = ep == kAccumulateF32;
  g.y_fastest = 1;
  if (w_layout == DG_LAYOUT_TILED)
    launch_gemm_bf16<true>(g, M, N, K, stream);
  else
    launch_gemm_bf16<false>(g, M, N, K, stream);
  DG_LAUNCH_CHECK();
  return DG_OK;
}

template <bool TILED>
static void launch_gemm_bf16(GemmArgs& g, int M, int N, int K, hipStream_t stream) {
  if (N >= 32768) {
    g.n_tiles_x = N / (64 * kWideRT);
    g.n_tiles_y = (M + 16 * kWideTB - 1) / (16 * kWideTB);
    g.n_tiles_total = g.n_tiles_x * g.n_tiles_y;
    gemm_stream_kernel<kWideRT, kWideTB, kWideKS, kWidePF, false, kDense, TILED>
        <<<(g.n_tiles_total + 7) / 8 * 8, 256, 0, stream>>>(g);
  } else if (K % 256 == 0 && N % 64 == 0) {
    // projections: 64 rows x 64 tokens per workgroup, K split over its waves
    // (16-token tiles when the output is too narrow to fill the chip)
    const bool narrow = N < 1024;
    g.n_tiles_x = N / 64;
    g.n_tiles_y = narrow ? (M + 15) / 16 : (M + 63) / 64;
    g.n_tiles_total = g.n_tiles_x * g.n_tiles_y;
    const unsigned grid = (g.n_tiles_total + 7) / 8 * 8;
    if (narrow)
      gemm_splitk_kernel<4, 1, kSplitNR, TILED><<<grid, 256, 0, stream>>>(g);
    else
      gemm_splitk_kernel<4, 4, kSplitNR, TILED><<<grid, 256, 0, stream>>>(g);
  } else {
    g.n_tiles_x = N / (64 * kDenseRT);
    g.n_tiles_y = (M + 16 * kDenseTB - 1) / (16 * kDenseTB);
    g.n_tiles_total = g.n_tiles_x * g.n_tiles_y;
    gemm_stream_kernel<kDenseRT, kDenseTB, kDenseKS, kDensePF, false, kDense, TILED>
        <<<(g.n_tiles_total + 7) / 8 * 8, 256, 0, stream>>>(g);
  }
}

template <typename TO>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ x,
                                                      TO* __restrict__ out, int D) {
  const int row = blockIdx.x;
  const float* xr = x + static_cast<int64_t>(row) * D;
  float ss = 0.f;
  for (int d = threadIdx.x; d < D; d += blockDim.x) ss = fmaf(xr[d], xr[d], ss);
  ss = warp_sum(ss);
  __shared__ float s_part[4];
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = s_part[0] + s_part[1] + s_part[2] + s_part[3];
  const float inv = rsqrtf(tot / D + 1e-6f);
  TO* o = out + static_cast<int64_t>(row) * D;
  for (int d = threadIdx.x; d < D; d += blockDim.x) Elem<TO>::store(o, d, xr[d] * inv);
}

dg_status launch_rmsnorm(const float* x, void* out, int M, int D, int out_dtype,
                         hipStream_t stream) {
  if (out_dtype == DG_BF16)
    rmsnorm_kernel<bf16_t><<<M, 256, 0, stream>>>(x, static_cast<bf16_t*>(out), D);
  else
    rmsnorm_kernel<float><<<M, 256, 0, stream>>>(x, static_cast<float*>(out), D);
  DG_LAUNCH_CHECK();
  return DG_OK;
}

template <typename T>
__global__ void embed_kernel(const int32_t* __restrict__ tokens, const T* __restrict__ emb,
                             float* __restrict__ x, int D) {
  const int row = blockIdx.x;
  const int64_t t = tokens[row];
  for (int d = threadIdx.x; d < D; d += blockDim.x)
    x[static_cast<int64_t>(row) * D + d] = Elem<T>::load(emb, t * D + d);
}

dg_status launch_embed(const int32_t* tokens, const void* emb, float* x, int M, int D, int dtype,
                       hipStream_t stream) {
  if (dtype == DG_BF16)
    embed_kernel<bf16_t><<<M, 256, 0, stream>>>(tokens, static_cast<const bf16_t*>(emb), x, D);
  else
    embed_kernel<float><<<M, 256, 0, stream>>>(tokens, static_cast<const float*>(emb), x, D);
  DG_LAUNCH_CHECK();
  return DG_OK;
}

}  // namespace dg
