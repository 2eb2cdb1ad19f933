// Dense projections (QKV, O, router, LM head), RMSNorm and the embedding
// gather of the decoder layer.
//
//   bf16: projections -- gemm_splitk_kernel (gemm_mfma.h), 128 weight rows x
//         32 tokens per workgroup (64 x 64 with tiled activations), K split
//         over its four waves;
//         LM head with tile-packed weights -- gemm_wide_kernel below;
//         other shapes -- gemm_stream_kernel in dense mode.
//   f32:  plain SIMT kernels (parity path of the tiny fp32 model).
// RMSNorm: x / sqrt(mean(x^2) + 1e-6), unit gain, f32 statistics.
#include "common.h"
#include "gemm_mfma.h"
#include "kernels.h"

namespace dg {

// projection-sized outputs (QKV, O, router): split-K register streaming,
// ring of kSplitNR chunks; wide outputs: 16 kProjRT rows x 16 kProjTB tokens
// per workgroup, K split over kProjNW waves; narrow outputs: 16 rows (router)
// or 32 rows (a handful of tokens) x 16 tokens, K split over eight waves
constexpr int kSplitNR = 2;
constexpr int kProjRT = 8, kProjTB = 2, kProjNW = 4, kProjWPE = 2;
// tiled activations: 64 rows x 64 tokens per workgroup (the least bytes per
// compute unit for these shapes: 720 KB against 900 KB at 256 tokens; QKV
// 14.4 -> 12.7 us, O 11.0 -> 9.3 us measured)
constexpr int kXtRT = 4, kXtTB = 4;
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

// Vocabulary-sized outputs with tile-packed weights (the LM head): one
// workgroup of 8 waves computes a 256-row x 256-token block of C^T, the
// weights read from HBM exactly once.  Per 64-k stage both operands pass
// through LDS (double buffered, staged in registers one stage ahead): the
// weight stage is the 16 tiles' packed 2 KB chunks copied as they are (the
// MFMA A-operand lane order), the token stage is 256 rows of 64 k with a
// 16-byte pad.  Wave (wr, wt) owns rows 128 wr .. +128 and tokens 64 wt ..
// +64: 32 accumulator blocks of 16 x 16, 12 KB of LDS reads per 32 MFMAs,
// below the LDS bandwidth at two waves per SIMD.
constexpr int kWideRows = 256, kWideTok = 256;
constexpr int kWideXStride = 64 + 8;                         // elements
constexpr int kWideWStage = kWideRows * 64;                  // elements
constexpr int kWideXStage = kWideTok * kWideXStride;         // elements
constexpr size_t kWideSmemBytes = 2 * (kWideWStage + kWideXStage) * sizeof(bf16_t);

// Registers of one stage: W pieces (four 16-byte pieces of the 16 tiles'
// packed chunks) and X pieces (token = item / 8, piece = item % 8; rows past
// M clamped).
struct WideStage {
  uint4 w0, w1, w2, w3, x0, x1, x2, x3;
};

__device__ __forceinline__ void wide_load_stage(WideStage& st, const bf16_t* wsrc,
                                                const bf16_t* X, int c, int K, int M, int m0,
                                                int tid) {
  auto wl = [&](int it) {
    const int item = it * 512 + tid;                   // 16-byte piece of the stage
    const int tile = item >> 7, piece = item & 127;    // 128 pieces per 2 KB chunk
    return *reinterpret_cast<const uint4*>(
        wsrc + (static_cast<int64_t>(tile) * (K / 64) + c) * 1024 + piece * 8);
  };
  auto xl = [&](int it) {
    const int item = it * 512 + tid;
    const int tok = min(m0 + (item >> 3), M - 1);
    return *reinterpret_cast<const uint4*>(X + static_cast<int64_t>(tok) * K + c * 64 + (item & 7) * 8);
  };
  st.w0 = wl(0); st.w1 = wl(1); st.w2 = wl(2); st.w3 = wl(3);
  st.x0 = xl(0); st.x1 = xl(1); st.x2 = xl(2); st.x3 = xl(3);
}

__device__ __forceinline__ void wide_store_stage(const WideStage& st, bf16_t* sw, bf16_t* sx,
                                                 int tid) {
  auto put = [&](int it, const uint4& w, const uint4& x) {
    const int item = it * 512 + tid;
    *reinterpret_cast<uint4*>(sw + item * 8) = w;
    *reinterpret_cast<uint4*>(sx + (item >> 3) * kWideXStride + (item & 7) * 8) = x;
  };
  put(0, st.w0, st.x0); put(1, st.w1, st.x1); put(2, st.w2, st.x2); put(3, st.w3, st.x3);
}

__global__ __launch_bounds__(512) void gemm_wide_kernel(const bf16_t* __restrict__ W,
                                                        const bf16_t* __restrict__ X,
                                                        bf16_t* __restrict__ C, int M, int N,
                                                        int K) {
  extern __shared__ __attribute__((aligned(16))) bf16_t wsm[];
  auto s_w = [&](int buf) { return wsm + buf * kWideWStage; };
  auto s_x = [&](int buf) { return wsm + 2 * kWideWStage + buf * kWideXStage; };
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int wr = wave & 1, wt = wave >> 1;
  const int n0 = blockIdx.x * kWideRows;
  const int m0 = blockIdx.y * kWideTok;
  const int nchunks = K / 64;

  const bf16_t* wsrc = W + static_cast<int64_t>(n0 / 16) * (K / 64) * 1024;
  WideStage st;
  f32x4_v acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_v{0.f, 0.f, 0.f, 0.f};

  wide_load_stage(st, wsrc, X, 0, K, M, m0, tid);
  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    wide_store_stage(st, s_w(buf), s_x(buf), tid);
    __syncthreads();
    if (c + 1 < nchunks) wide_load_stage(st, wsrc, X, c + 1, K, M, m0, tid);
    const bf16_t* sw = s_w(buf) + wr * 8 * 1024;
    const bf16_t* sx = s_x(buf) + (wt * 64) * kWideXStride;
#pragma unroll
    for (int h = 0; h < 2; ++h) {            // the two 8-value halves of a lane's 16 k
      bf16x8_v xb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        xb[j] = *reinterpret_cast<const bf16x8_v*>(sx + (j * 16 + l16) * kWideXStride + g4 * 16 + h * 8);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bf16x8_v wa = *reinterpret_cast<const bf16x8_v*>(sw + i * 1024 + h * 512 + lane * 8);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, xb[j], acc[i][j], 0, 0, 0);
      }
    }
  }

  // epilogue: lane holds rows 4 g4 + r of row tile i, token l16 of block j
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + wt * 64 + j * 16 + l16;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int n = n0 + wr * 128 + i * 16 + g4 * 4;
      uint2 pk;
      pk.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
      pk.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
      *reinterpret_cast<uint2*>(C + static_cast<int64_t>(m) * N + n) = pk;
    }
  }
}

// The same block GEMM with both operands copied global -> LDS by the
// direct-to-LDS 16-byte loads (global_load_lds_dwordx4: lane l of a wave
// instruction writes LDS bytes [16 l, 16 l + 16) after the instruction's
// base, from any global address), so no registers hold a stage in flight
// and the weights run two stages ahead: 3 weight buffers (32 KB each) and 2
// token buffers (32 KB each, unpadded, 16-byte pieces XOR-swizzled by row so
// the B-operand reads spread over the banks).
constexpr int kDlWStages = 3, kDlXStages = 2;
constexpr bool kWideDirectLds = true;   // LM head: direct-to-LDS form
constexpr size_t kDlSmemBytes = (kDlWStages * kWideWStage + kDlXStages * kWideTok * 64) * sizeof(bf16_t);

__device__ __forceinline__ int dl_xslot(int row, int piece) { return piece ^ ((row >> 1) & 7); }

constexpr int kWaitVm4 = waitcnt_vm(4), kWaitVm0 = waitcnt_vm(0);

__global__ __launch_bounds__(512) void gemm_wide_dl_kernel(const bf16_t* __restrict__ W,
                                                           const bf16_t* __restrict__ X,
                                                           bf16_t* __restrict__ C, int M, int N,
                                                           int K, const int32_t* gate,
                                                           int gate_n) {
  extern __shared__ __attribute__((aligned(16))) bf16_t dsm[];
  if (step_gate_closed(gate, gate_n)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int wr = wave & 1, wt = wave >> 1;
  // logical tile: token tiles of one row tile adjacent, and each XCD a
  // contiguous range, so the token tiles of a weight tile (more than 256
  // tokens) read it into one L2 once
  const int mt = (M + kWideTok - 1) / kWideTok;
  const int total = (N / kWideRows) * mt;
  const int logical = xcd_logical_tile(blockIdx.x, gridDim.x);
  if (logical >= total) return;
  const int n0 = (logical / mt) * kWideRows;
  const int m0 = (logical % mt) * kWideTok;
  const int nchunks = K / 64;
  const bf16_t* wsrc = W + static_cast<int64_t>(n0 / 16) * (K / 64) * 1024;

  // wave w copies 1 KB blocks 4w .. 4w + 3 of each stage
  auto issue_w = [&](int c) {            // weight stage c -> buffer c % 3
    bf16_t* dst = dsm + (c % kDlWStages) * kWideWStage;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = wave * 4 + i;         // block: tile b / 2, half b % 2
      const bf16_t* src = wsrc + (static_cast<int64_t>(b >> 1) * (K / 64) + c) * 1024 +
                          (b & 1) * 512 + lane * 8;
      __builtin_amdgcn_global_load_lds(src, dst + b * 512, 16, 0, 0);
    }
  };
  auto issue_x = [&](int c) {            // token stage c -> buffer c % 2
    bf16_t* dst = dsm + kDlWStages * kWideWStage + (c % kDlXStages) * kWideTok * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = wave * 4 + i;         // rows 8 b .. 8 b + 7
      const int row = b * 8 + (lane >> 3);
      const int piece = (lane & 7) ^ ((row >> 1) & 7);   // slot lane & 7 holds this piece
      const int tok = min(m0 + row, M - 1);
      const bf16_t* src = X + static_cast<int64_t>(tok) * K + c * 64 + piece * 8;
      __builtin_amdgcn_global_load_lds(src, dst + b * 512, 16, 0, 0);
    }
  };

  f32x4_v acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_v{0.f, 0.f, 0.f, 0.f};

  // prologue: W(0), X(0), W(1); iteration c issues X(c + 1), W(c + 2)
  issue_w(0);
  issue_x(0);
  if (nchunks > 1) issue_w(1);
  for (int c = 0; c < nchunks; ++c) {
    // stage c's loads are done when at most W(c + 1)'s four are outstanding
    if (c + 1 < nchunks) __builtin_amdgcn_s_waitcnt(kWaitVm4);
    else __builtin_amdgcn_s_waitcnt(kWaitVm0);
    // every wave's copies landed (each waited for its own above); stage c - 1
    // consumed.  A bare barrier: the fence of __syncthreads would wait for
    // the stages still in flight as well.
    __builtin_amdgcn_s_barrier();
    if (c + 1 < nchunks) issue_x(c + 1);
    if (c + 2 < nchunks) issue_w(c + 2);
    const bf16_t* sw = dsm + (c % kDlWStages) * kWideWStage + wr * 8 * 1024;
    const bf16_t* sx = dsm + kDlWStages * kWideWStage + (c % kDlXStages) * kWideTok * 64;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x8_v xb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = wt * 64 + j * 16 + l16;
        xb[j] = *reinterpret_cast<const bf16x8_v*>(sx + row * 64 + dl_xslot(row, g4 * 2 + h) * 8);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bf16x8_v wa = *reinterpret_cast<const bf16x8_v*>(sw + i * 1024 + h * 512 + lane * 8);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, xb[j], acc[i][j], 0, 0, 0);
      }
    }
  }

#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + wt * 64 + j * 16 + l16;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int n = n0 + wr * 128 + i * 16 + g4 * 4;
      uint2 pk;
      pk.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
      pk.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
      *reinterpret_cast<uint2*>(C + static_cast<int64_t>(m) * N + n) = pk;
    }
  }
}

template <bool TILED>
static dg_status launch_gemm_bf16(GemmArgs& g, int M, int N, int K, hipStream_t stream);

dg_status launch_gemm(const void* A, const void* W, void* C, int M, int N, int K, int dtype,
                      int w_layout, int out_dtype, GemmEpilogue ep, hipStream_t stream,
                      const StepGate& gate) {
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
  g.gate = gate.n_done;
  g.gate_n = gate.n;
  const dg_status st = w_layout == DG_LAYOUT_TILED ? launch_gemm_bf16<true>(g, M, N, K, stream)
                                                    : launch_gemm_bf16<false>(g, M, N, K, stream);
  if (st != DG_OK) return st;
  DG_LAUNCH_CHECK();
  return DG_OK;
}

// A thousand tokens and more with tiled activations: 128 x 128 tiles staged
// through LDS (gemm_dl128_kernel).  Stages in flight: 4 (128 KB of LDS, one
// workgroup per CU) while the grid fits the 256 CUs once, else 2 (64 KB, two
// workgroups per CU).  Measured at 2048 / 1024 tokens against the split-K
// tiles: QKV 111 -> 52 / 48 -> 33 us, O 64 -> 38 / 30 -> 29 us (O at 2048
// tokens, 352 tiles: 54 us with four stages).
constexpr int kDl128MinTokens = 1024;

static dg_status launch_dl128(GemmArgs& g, int M, int N, hipStream_t stream) {
  g.n_tiles_x = N / 128;
  g.n_tiles_y = (M + 127) / 128;
  g.n_tiles_total = g.n_tiles_x * g.n_tiles_y;
  const unsigned grid = (g.n_tiles_total + 7) / 8 * 8;
  if (g.n_tiles_total > 256) {
    constexpr int kBytes = 2 * kDl128Stage * static_cast<int>(sizeof(bf16_t));
    gemm_dl128_kernel<2><<<grid, 256, kBytes, stream>>>(g);
  } else {
    constexpr int kBytes = 4 * kDl128Stage * static_cast<int>(sizeof(bf16_t));
    const dg_status st = ensure_lds_limit(reinterpret_cast<const void*>(gemm_dl128_kernel<4>), kBytes);
    if (st != DG_OK) return st;
    gemm_dl128_kernel<4><<<grid, 256, kBytes, stream>>>(g);
  }
  DG_LAUNCH_CHECK();
  return DG_OK;
}

bool qkv_rope_supported(const QkvRope& r, int K) {
  const int M = r.B * r.Lq;
  const int N = (r.Hq + 2 * r.Hkv) * r.dh;
  // the wide split-K tiles: 16 kProjRT = 128 rows = one head of 128 (tiled
  // activations: 64-row tiles, half a head's rotated pairs each); a handful
  // of tokens (AR decode): 32-row tiles, a quarter of a head's pairs each
  return r.dh == 128 && kProjRT == 8 && kXtRT == 4 && M >= 1 && N >= 1024 && K % 64 == 0 &&
         K >= 64 * 8 && r.Hq % r.Hkv == 0 && (M > 16 || !r.x_tiled);
}

bool dense_xt_supported(int M, int N, int K) {
  return M > 16 && N % (16 * kXtRT) == 0 && K % 64 == 0 && K >= 64 * 8;
}

dg_status launch_qkv_rope(const void* A, const void* W, int K, int w_layout, const QkvRope& r,
                          hipStream_t stream, const StepGate& gate) {
  const int M = r.B * r.Lq;
  const int N = (r.Hq + 2 * r.Hkv) * r.dh;
  if (!qkv_rope_supported(r, K) || (r.x_tiled && w_layout != DG_LAYOUT_TILED))
    return DG_ERR_UNSUPPORTED;
  if (!r.rope_tab) return DG_ERR_INVALID_ARG;
  GemmArgs g{};
  g.W = W; g.X = static_cast<const bf16_t*>(A);
  g.N = N; g.K = K; g.M = M; g.n_groups = 1;
  g.out_dtype = DG_BF16;
  g.y_fastest = 1;
  g.rope = 1;
  g.prefix_len = r.prefix_len;
  g.Lq = r.Lq; g.Hq = r.Hq; g.Hkv = r.Hkv; g.Tmax = r.Tmax;
  g.q_scale = attn_q_scale(r.dh);
  g.rope_tab = r.rope_tab;
  g.q_out = static_cast<bf16_t*>(r.q_out);
  g.k_cache = static_cast<bf16_t*>(r.k_cache);
  g.v_cache = static_cast<bf16_t*>(r.v_cache);
  g.x_tiled = r.x_tiled;
  g.gate = gate.n_done;
  g.gate_n = gate.n;
  if (r.x_tiled && M >= kDl128MinTokens) return launch_dl128(g, M, N, stream);
  if (M <= 16) {
    // the narrow split-K tiles of a handful of tokens (32 weight rows, eight
    // waves over K), RoPE in their epilogue instead of a separate kernel
    g.n_tiles_x = N / 32;
    g.n_tiles_y = 1;
    g.n_tiles_total = g.n_tiles_x;
    const unsigned grid = (g.n_tiles_total + 7) / 8 * 8;
    if (w_layout == DG_LAYOUT_TILED)
      gemm_splitk_kernel<2, 1, kSplitNR, 8, true><<<grid, 512, 0, stream>>>(g);
    else
      gemm_splitk_kernel<2, 1, kSplitNR, 8, false><<<grid, 512, 0, stream>>>(g);
    DG_LAUNCH_CHECK();
    return DG_OK;
  }
  const int rt = r.x_tiled ? kXtRT : kProjRT, tb = r.x_tiled ? kXtTB : kProjTB;
  g.n_tiles_x = N / (16 * rt);
  g.n_tiles_y = (M + 16 * tb - 1) / (16 * tb);
  g.n_tiles_total = g.n_tiles_x * g.n_tiles_y;
  const unsigned grid = (g.n_tiles_total + 7) / 8 * 8;
  if (r.x_tiled)
    gemm_splitk_kernel<kXtRT, kXtTB, kSplitNR, kProjNW, true, kProjWPE>
        <<<grid, 64 * kProjNW, 0, stream>>>(g);
  else if (w_layout == DG_LAYOUT_TILED)
    gemm_splitk_kernel<kProjRT, kProjTB, kSplitNR, kProjNW, true, kProjWPE>
        <<<grid, 64 * kProjNW, 0, stream>>>(g);
  else
    gemm_splitk_kernel<kProjRT, kProjTB, kSplitNR, kProjNW, false, kProjWPE>
        <<<grid, 64 * kProjNW, 0, stream>>>(g);
  DG_LAUNCH_CHECK();
  return DG_OK;
}

dg_status launch_gemm_xt(const void* A, const void* W, void* C, int M, int N, int K,
                         int out_dtype, GemmEpilogue ep, hipStream_t stream,
                         const StepGate& gate) {
  if (!dense_xt_supported(M, N, K) || (out_dtype != DG_BF16 && out_dtype != DG_F32) ||
      (ep == kAccumulateF32 && out_dtype != DG_F32))
    return DG_ERR_UNSUPPORTED;
  GemmArgs g{};
  g.W = W; g.X = static_cast<const bf16_t*>(A); g.out = C;
  g.N = N; g.K = K; g.M = M; g.n_groups = 1;
  g.out_dtype = out_dtype;
  g.accumulate = ep == kAccumulateF32;
  g.y_fastest = 1;
  g.x_tiled = 1;
  g.gate = gate.n_done;
  g.gate_n = gate.n;
  if (M >= kDl128MinTokens && N % 128 == 0) return launch_dl128(g, M, N, stream);
  g.n_tiles_x = N / (16 * kXtRT);
  g.n_tiles_y = (M + 16 * kXtTB - 1) / (16 * kXtTB);
  g.n_tiles_total = g.n_tiles_x * g.n_tiles_y;
  gemm_splitk_kernel<kXtRT, kXtTB, kSplitNR, kProjNW, true, kProjWPE>
      <<<(g.n_tiles_total + 7) / 8 * 8, 64 * kProjNW, 0, stream>>>(g);
  DG_LAUNCH_CHECK();
  return DG_OK;
}

template <bool TILED>
static dg_status launch_gemm_bf16(GemmArgs& g, int M, int N, int K, hipStream_t stream) {
  // wide outputs (the LM head) over many tokens: 256 x 256 tiles staged
  // through LDS; over a handful of tokens (AR decode) the split-K streaming
  // tiles below move the weights faster (6.0 against 3.7 TB/s at one token)
  if (TILED && M > 16 && N >= 32768 && N % kWideRows == 0 && K % 64 == 0 && !g.accumulate &&
      g.out_dtype == DG_BF16) {
    dg_status lst = ensure_lds_limit(reinterpret_cast<const void*>(gemm_wide_kernel),
                                     static_cast<int>(kWideSmemBytes));
    if (lst == DG_OK)
      lst = ensure_lds_limit(reinterpret_cast<const void*>(gemm_wide_dl_kernel),
                             static_cast<int>(kDlSmemBytes));
    if (lst != DG_OK) return lst;
    dim3 grid(N / kWideRows, (M + kWideTok - 1) / kWideTok);
    const unsigned dl_grid = (grid.x * grid.y + 7) / 8 * 8;
    if (kWideDirectLds)
      gemm_wide_dl_kernel<<<dl_grid, 512, kDlSmemBytes, stream>>>(
          static_cast<const bf16_t*>(g.W), g.X, static_cast<bf16_t*>(g.out), M, N, K, g.gate,
          g.gate_n);
    else
      gemm_wide_kernel<<<grid, 512, kWideSmemBytes, stream>>>(
          static_cast<const bf16_t*>(g.W), g.X, static_cast<bf16_t*>(g.out), M, N, K);
  } else if (M > 16 && N >= 32768 && N % (64 * kWideRT) == 0) {
    g.n_tiles_x = N / (64 * kWideRT);
    g.n_tiles_y = (M + 16 * kWideTB - 1) / (16 * kWideTB);
    g.n_tiles_total = g.n_tiles_x * g.n_tiles_y;
    gemm_stream_kernel<kWideRT, kWideTB, kWideKS, kWidePF, kWBf16, kDense, TILED>
        <<<(g.n_tiles_total + 7) / 8 * 8, 256, 0, stream>>>(g);
  } else if (K % 64 == 0 && K >= 64 * 8 && N % (16 * kProjRT) == 0 && N % 32 == 0) {
    // narrow outputs, or a handful of tokens (AR decode): more, smaller tiles
    // (router outputs: 16-row tiles; a few tokens: 32-row tiles)
    const bool narrow = N < 1024 || M <= 16;
    const int narrow_rows = N < 1024 ? 16 : 32;
    g.n_tiles_x = narrow ? N / narrow_rows : N / (16 * kProjRT);
    g.n_tiles_y = narrow ? (M + 15) / 16 : (M + 16 * kProjTB - 1) / (16 * kProjTB);
    g.n_tiles_total = g.n_tiles_x * g.n_tiles_y;
    const unsigned grid = (g.n_tiles_total + 7) / 8 * 8;
    if (narrow && narrow_rows == 16)
      gemm_splitk_kernel<1, 1, kSplitNR, 8, TILED><<<grid, 512, 0, stream>>>(g);
    else if (narrow)
      gemm_splitk_kernel<2, 1, kSplitNR, 8, TILED><<<grid, 512, 0, stream>>>(g);
    else
      gemm_splitk_kernel<kProjRT, kProjTB, kSplitNR, kProjNW, TILED, kProjWPE>
          <<<grid, 64 * kProjNW, 0, stream>>>(g);
  } else {
    g.n_tiles_x = N / (64 * kDenseRT);
    g.n_tiles_y = (M + 16 * kDenseTB - 1) / (16 * kDenseTB);
    g.n_tiles_total = g.n_tiles_x * g.n_tiles_y;
    gemm_stream_kernel<kDenseRT, kDenseTB, kDenseKS, kDensePF, kWBf16, kDense, TILED>
        <<<(g.n_tiles_total + 7) / 8 * 8, 256, 0, stream>>>(g);
  }
  return DG_OK;
}

// One row per workgroup; the row stays in registers (float4 pieces) between
// the sum of squares and the scaled store, so x is read once.
constexpr int kNormPieces = 4;     // float4 pieces per thread: D <= 4096

// With y_slot, the row first takes the MoE combine: x += sum_j y_slot[row *
// k + j] in slot order, and the updated row is written back.  Every load is
// issued unconditionally from a clamped address and masked afterwards, so the
// loads of a row stay in flight together.
template <typename TS> struct Slot4;
template <> struct Slot4<bf16_t> {
  uint2 u;
  __device__ void load(const bf16_t* p) { u = *reinterpret_cast<const uint2*>(p); }
  __device__ float4 get() const {
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
  }
};
template <> struct Slot4<float> {
  float4 f;
  __device__ void load(const float* p) { f = *reinterpret_cast<const float4*>(p); }
  __device__ float4 get() const { return f; }
};

// (cos, sin) of row `row`'s RoPE pairs into rt.tab (threads j < rt.pairs)
__device__ __forceinline__ void rope_table_row(const RopeTable& rt, int row) {
  const int j = threadIdx.x;
  if (rt.tab == nullptr || j >= rt.pairs) return;
  const int pos = rt.prefix_len[row / rt.Lq] + row % rt.Lq;
  float c, s;
  rope_cos_sin(pos, j, 2 * rt.pairs, rt.theta, &c, &s);
  rt.tab[static_cast<int64_t>(row) * rt.pairs + j] = make_float2(c, s);
}

__device__ __forceinline__ int norm_in_row(const NormRows& nr, int r) {
  return nr.blk > 0 ? (r / nr.blk) * nr.in_blk + nr.in_off + r % nr.blk : r;
}

template <typename TS, typename TO>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const TS* __restrict__ y_slot, int k,
                                                      float* __restrict__ x,
                                                      TO* __restrict__ out, int D, int tiled,
                                                      RopeTable rt, NormRows nr) {
  const int orow = blockIdx.x;                  // output row
  const int row = norm_in_row(nr, orow);        // input row of x (and y_slot)
  rope_table_row(rt, row);
  float4* xr = reinterpret_cast<float4*>(x + static_cast<int64_t>(row) * D);
  const int n4 = D / 4;
  float4 v[kNormPieces];
#pragma unroll
  for (int i = 0; i < kNormPieces; ++i) v[i] = xr[min(i * 256 + static_cast<int>(threadIdx.x), n4 - 1)];
  if (y_slot) {
    // slots in groups of 8: loads of a group in flight together, added in order
    for (int j0 = 0; j0 < k; j0 += 8) {
      Slot4<TS> sv[kNormPieces][8];
#pragma unroll
      for (int i = 0; i < kNormPieces; ++i) {
        const int p = min(i * 256 + static_cast<int>(threadIdx.x), n4 - 1);
#pragma unroll
        for (int u = 0; u < 8; ++u)
          sv[i][u].load(y_slot + (static_cast<int64_t>(row) * k + min(j0 + u, k - 1)) * D + 4 * p);
      }
#pragma unroll
      for (int i = 0; i < kNormPieces; ++i)
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (j0 + u < k) {
            const float4 a = sv[i][u].get();
            v[i].x += a.x;
            v[i].y += a.y;
            v[i].z += a.z;
            v[i].w += a.w;
          }
        }
    }
#pragma unroll
    for (int i = 0; i < kNormPieces; ++i) {
      const int p = i * 256 + threadIdx.x;
      if (p < n4) xr[p] = v[i];
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kNormPieces; ++i) {
    const int p = i * 256 + threadIdx.x;
    if (p >= n4) v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    ss = fmaf(v[i].x, v[i].x, fmaf(v[i].y, v[i].y, fmaf(v[i].z, v[i].z, fmaf(v[i].w, v[i].w, ss))));
  }
  ss = warp_sum(ss);
  __shared__ float s_part[4];
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = s_part[0] + s_part[1] + s_part[2] + s_part[3];
  const float inv = rsqrtf(tot / D + 1e-6f);
  TO* o = out + static_cast<int64_t>(orow) * D;
#pragma unroll
  for (int i = 0; i < kNormPieces; ++i) {
    const int p = i * 256 + threadIdx.x;
    if (p >= n4) continue;
    if constexpr (sizeof(TO) == 2) {
      uint2 pk;
      pk.x = pack_bf16x2(v[i].x * inv, v[i].y * inv);
      pk.y = pack_bf16x2(v[i].z * inv, v[i].w * inv);
      TO* dst = tiled ? out + xtile_offset(orow, 4 * p, D) : o + 4 * p;
      *reinterpret_cast<uint2*>(dst) = pk;
    } else {
      *reinterpret_cast<float4*>(o + 4 * p) =
          make_float4(v[i].x * inv, v[i].y * inv, v[i].z * inv, v[i].w * inv);
    }
  }
}

// Rows wider than the register-resident kernel holds, or not a multiple of 4.
template <typename TO>
__global__ __launch_bounds__(256) void rmsnorm_wide_kernel(const float* __restrict__ x,
                                                           TO* __restrict__ out, int D,
                                                           RopeTable rt, NormRows nr) {
  const int orow = blockIdx.x;
  const int row = norm_in_row(nr, orow);
  rope_table_row(rt, row);
  const float* xr = x + static_cast<int64_t>(row) * D;
  float ss = 0.f;
  for (int d = threadIdx.x; d < D; d += blockDim.x) ss = fmaf(xr[d], xr[d], ss);
  ss = warp_sum(ss);
  __shared__ float s_part[4];
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = s_part[0] + s_part[1] + s_part[2] + s_part[3];
  const float inv = rsqrtf(tot / D + 1e-6f);
  TO* o = out + static_cast<int64_t>(orow) * D;
  for (int d = threadIdx.x; d < D; d += blockDim.x) Elem<TO>::store(o, d, xr[d] * inv);
}

dg_status launch_rmsnorm(const float* x, void* out, int M, int D, int out_dtype,
                         hipStream_t stream) {
  return launch_combine_rmsnorm(nullptr, DG_BF16, 0, const_cast<float*>(x), out, M, D, out_dtype,
                                stream);
}

dg_status launch_combine_rmsnorm(const void* y_slot, int slot_dtype, int k, float* x, void* out,
                                 int M, int D, int out_dtype, hipStream_t stream, bool out_tiled,
                                 const RopeTable& rope, const NormRows& rows) {
  if (rope.tab && (rope.pairs <= 0 || rope.pairs > 256 || rope.Lq <= 0 || !rope.prefix_len))
    return DG_ERR_INVALID_ARG;
  if (rows.blk < 0 || (rows.blk > 0 && (rows.in_off < 0 || rows.in_off + rows.blk > rows.in_blk)))
    return DG_ERR_INVALID_ARG;
  const bool regs = D % 4 == 0 && D / 4 <= kNormPieces * 256;
  if (out_tiled && !(regs && D % 64 == 0 && out_dtype == DG_BF16)) return DG_ERR_UNSUPPORTED;
  const int tl = out_tiled ? 1 : 0;
  if (!regs) {
    if (rows.blk > 0) return DG_ERR_UNSUPPORTED;   // the row map needs the fused combine
    dg_status st;
    if (y_slot && (st = launch_moe_combine(y_slot, slot_dtype, M, D, k, x, stream))) return st;
    if (out_dtype == DG_BF16)
      rmsnorm_wide_kernel<bf16_t><<<M, 256, 0, stream>>>(x, static_cast<bf16_t*>(out), D, rope, rows);
    else
      rmsnorm_wide_kernel<float><<<M, 256, 0, stream>>>(x, static_cast<float*>(out), D, rope, rows);
    DG_LAUNCH_CHECK();
    return DG_OK;
  }
  const bool bf = slot_dtype == DG_BF16;
  const bf16_t* yb = bf ? static_cast<const bf16_t*>(y_slot) : nullptr;
  const float* yf = bf ? nullptr : static_cast<const float*>(y_slot);
  if (out_dtype == DG_BF16) {
    if (bf) rmsnorm_kernel<bf16_t, bf16_t><<<M, 256, 0, stream>>>(yb, k, x, static_cast<bf16_t*>(out), D, tl, rope, rows);
    else rmsnorm_kernel<float, bf16_t><<<M, 256, 0, stream>>>(yf, k, x, static_cast<bf16_t*>(out), D, tl, rope, rows);
  } else {
    if (bf) rmsnorm_kernel<bf16_t, float><<<M, 256, 0, stream>>>(yb, k, x, static_cast<float*>(out), D, 0, rope, rows);
    else rmsnorm_kernel<float, float><<<M, 256, 0, stream>>>(yf, k, x, static_cast<float*>(out), D, 0, rope, rows);
  }
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
