// Dense projections (QKV, O, router, LM head), RMSNorm and the embedding
// gather of the decoder layer.
//
//   bf16: gemm_stream_kernel (gemm_mfma.h) in dense mode -- weights streamed
//         once per 128-token tile, tokens staged in LDS.
//   f32:  plain SIMT kernels (parity path of the tiny fp32 model).
// RMSNorm: x / sqrt(mean(x^2) + 1e-6), unit gain, f32 statistics.
#include "common.h"
#include "gemm_mfma.h"
#include "kernels.h"

namespace dg {

constexpr int kDenseTB = 8;    // 128 tokens per tile
constexpr int kDenseKS = 2;    // 128 k per LDS stage

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

dg_status launch_gemm(const void* A, const void* W, void* C, int M, int N, int K, int dtype,
                      int out_dtype, GemmEpilogue ep, hipStream_t stream) {
  if (dtype == DG_F32) {
    dim3 grid((N + 127) / 128, M);
    gemm_f32_kernel<<<grid, 128, 0, stream>>>(static_cast<const float*>(A),
                                              static_cast<const float*>(W),
                                              static_cast<float*>(C), M, N, K,
                                              ep == kAccumulateF32);
    DG_LAUNCH_CHECK();
    return DG_OK;
  }
  constexpr int MT = 16 * kDenseTB;
  GemmArgs g{};
  g.W = W; g.X = static_cast<const bf16_t*>(A);
  g.N = N; g.K = K; g.M = M; g.n_groups = 1;
  g.out = C;
  g.out_dtype = ep == kAccumulateF32 ? DG_F32 : out_dtype;
  g.accumulate = ep == kAccumulateF32;
  g.n_tiles_x = N / 128;
  g.n_tiles_total = g.n_tiles_x * ((M + MT - 1) / MT);
  gemm_stream_kernel<2, kDenseTB, kDenseKS, false, kDense>
      <<<(g.n_tiles_total + 7) / 8 * 8, 256, 0, stream>>>(g);
  DG_LAUNCH_CHECK();
  return DG_OK;
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
