// Weight-streaming MFMA GEMM for small token counts (gfx950).
//
//   out[token, row] = sum_k W[row, k] * X[token, k]      (W: [N, K] row-major)
//
// The weights are the stream that matters (each byte is read from HBM once
// per token tile); the token count per tile is small (16..128).  So the
// weights are the MFMA A operand and live only in registers: a wave owns
// RT tiles of 16 weight rows and keeps a ring of KS chunks (64 k each) of
// them in flight, one full LDS stage ahead.  The tokens are the B operand:
// the workgroup copies a stage of KS * 64 k of its MT = 16 * TB token rows
// into LDS once (double buffered) and every wave reads its fragments there.
//
// Per 64-k chunk a lane holds 16 consecutive k of its row (16 B of fp8 or
// 32 B of bf16 starting at 16 * (lane / 16)); the two v_mfma_f32_16x16x32_bf16
// of the chunk take its first and second 8 values.  The token fragments use
// the same k order, so the products pair up.  fp8 (OCP e4m3fn) weights are
// widened to bf16 exactly in registers; their per-row scale is applied in the
// epilogue, where it factors out of the sum.
//
// Modes:
//   kGateUp  rows of tile 0 = gate rows n0 + 16 wave + i, tile 1 = up rows
//            I + n0 + ...; epilogue h = GELU_erf(s_g acc0) * (s_u acc1) -> bf16
//            h[sorted position, n]; tokens are the slots of one expert.
//   kDown    A rows = W_down rows; X = h rows in sorted order; epilogue
//            y_slot[slot, row] = gate[slot] * s * acc (f32).
//   kDense   one group; X rows = tokens; epilogue stores (bf16 / f32) or adds
//            into an f32 output.
#pragma once

#include "common.h"

namespace dg {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_v;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_v;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_v;

enum GemmMode { kGateUp = 0, kDown = 1, kDense = 2 };

struct GemmArgs {
  const void* W;            // weights (bf16 or fp8 bytes)
  int64_t w_group_stride;   // elements between experts
  const float* w_scale;     // per-row scale (fp8) or null
  int64_t s_group_stride;
  const bf16_t* X;          // activations [rows, K] bf16
  int N;                    // rows per group (gate_up: 2I; down: D; dense: N)
  int K;
  int M;                    // dense: token count
  int n_groups;             // experts (1 for dense)
  int topk;                 // slots per token (grouped modes)
  const int32_t* offsets;   // [E + 1] (grouped)
  const int32_t* sorted_rows;
  const float* gates;       // [T * k]
  void* out;                // gate_up: h bf16 [T*k, I]; down: y_slot f32 [T*k, D];
                            // dense: [M, N] in out_dtype
  int out_dtype;            // dense: DG_BF16 / DG_F32
  int accumulate;           // dense: out (f32) += result
  int n_tiles_x;            // row tiles per group
  int n_tiles_total;        // logical workgroups (x * y)
};

__device__ __forceinline__ float gelu_erf(float x) {
  return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
}

// 16 fp8 (OCP e4m3fn) bytes -> two bf16x8 (exact widening).
__device__ __forceinline__ void fp8x16_to_bf16(const uint4& q, bf16x8_v& lo, bf16x8_v& hi) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  bf16x2_v p[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p[2 * i] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w[i]), 1.0f, false);
    p[2 * i + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w[i]), 1.0f, true);
  }
  lo = bf16x8_v{p[0][0], p[0][1], p[1][0], p[1][1], p[2][0], p[2][1], p[3][0], p[3][1]};
  hi = bf16x8_v{p[4][0], p[4][1], p[5][0], p[5][1], p[6][0], p[6][1], p[7][0], p[7][1]};
}

template <bool FP8> struct WChunk;
template <> struct WChunk<true> {
  uint4 q;
  __device__ void load(const uint8_t* p) { q = *reinterpret_cast<const uint4*>(p); }
  __device__ void zero() { q = make_uint4(0, 0, 0, 0); }
  __device__ void get(bf16x8_v& a, bf16x8_v& b) const { fp8x16_to_bf16(q, a, b); }
};
template <> struct WChunk<false> {
  uint4 q0, q1;
  __device__ void load(const bf16_t* p) {
    q0 = *reinterpret_cast<const uint4*>(p);
    q1 = *reinterpret_cast<const uint4*>(p + 8);
  }
  __device__ void zero() { q0 = q1 = make_uint4(0, 0, 0, 0); }
  __device__ void get(bf16x8_v& a, bf16x8_v& b) const {
    a = *reinterpret_cast<const bf16x8_v*>(&q0);
    b = *reinterpret_cast<const bf16x8_v*>(&q1);
  }
};

// Logical workgroup index: consecutive logical tiles go to the same XCD
// (hardware dispatches linear workgroup ids round-robin over 8 XCDs), so the
// row tiles that share a token tile share that XCD's L2.
__device__ __forceinline__ int xcd_logical_tile(int linear, int total) {
  const int per = (total + 7) / 8;
  return (linear % 8) * per + linear / 8;
}

template <int RT, int TB, int KS, bool FP8, int MODE>
__global__ __launch_bounds__(256) void gemm_stream_kernel(GemmArgs a) {
  using WT = typename std::conditional<FP8, uint8_t, bf16_t>::type;
  constexpr int MT = 16 * TB;           // tokens per tile
  constexpr int SK = 64 * KS;           // k per LDS stage
  constexpr int XS = SK + 8;            // LDS row stride (elements)
  __shared__ __attribute__((aligned(16))) bf16_t s_x[2][MT * XS];
  __shared__ int s_rows[MT];            // source row of each token of the tile
  __shared__ int s_dst[MT];             // destination row (grouped modes)
  __shared__ int s_scan[256];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int logical = xcd_logical_tile(blockIdx.x, gridDim.x);
  if (logical >= a.n_tiles_total) return;
  const int tx = logical % a.n_tiles_x;       // row tile within the group
  const int ty = logical / a.n_tiles_x;       // token-tile slot

  // ---- which group / token range this tile covers
  int grp = 0, m0 = 0, m_count = 0, base_pos = 0;
  if (MODE == kDense) {
    m0 = ty * MT;
    if (m0 >= a.M) return;
    m_count = min(MT, a.M - m0);
  } else {
    const int E = a.n_groups;
    int tiles_e = 0;
    if (tid < E) tiles_e = (a.offsets[tid + 1] - a.offsets[tid] + MT - 1) / MT;
    s_scan[tid] = tiles_e;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {        // inclusive scan over <= 256 groups
      const int v = (tid >= o) ? s_scan[tid - o] : 0;
      __syncthreads();
      s_scan[tid] += v;
      __syncthreads();
    }
    if (ty >= s_scan[E - 1]) return;
    int lo = 0, hi = E - 1;                    // first e with scan[e] > ty
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_scan[mid] > ty) hi = mid; else lo = mid + 1;
    }
    grp = lo;
    const int first_tile = grp ? s_scan[grp - 1] : 0;
    base_pos = a.offsets[grp];
    m0 = (ty - first_tile) * MT;
    m_count = min(MT, a.offsets[grp + 1] - base_pos - m0);
  }
  if (tid < MT) {
    int src = -1, dst = -1;
    if (tid < m_count) {
      const int m = m0 + tid;
      if (MODE == kDense) { src = m; dst = m; }
      else if (MODE == kGateUp) { const int p = base_pos + m; src = a.sorted_rows[p] / a.topk; dst = p; }
      else { const int p = base_pos + m; src = p; dst = a.sorted_rows[p]; }
    }
    s_rows[tid] = src;
    s_dst[tid] = dst;
  }
  __syncthreads();

  // ---- weight rows of this wave
  const WT* Wg = static_cast<const WT*>(a.W) + static_cast<int64_t>(grp) * a.w_group_stride;
  int wrow[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    if (MODE == kGateUp) wrow[rt] = (rt == 0 ? 0 : a.N / 2) + tx * 64 + wave * 16 + l16;
    else wrow[rt] = tx * (64 * RT) + wave * (16 * RT) + rt * 16 + l16;
  }
  const int nchunks = (a.K + 63) / 64;
  const int nstages = (nchunks + KS - 1) / KS;

  WChunk<FP8> wr[KS][RT];
  auto load_w = [&](int stage) {
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      const int c = stage * KS + j;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        if (c < nchunks && wrow[rt] < a.N)
          wr[j][rt].load(Wg + static_cast<int64_t>(wrow[rt]) * a.K + c * 64 + g4 * 16);
        else
          wr[j][rt].zero();
      }
    }
  };
  auto stage_x = [&](int stage, int buf) {
    // MT rows x SK k of bf16: 16-byte pieces, SK / 8 per row
    constexpr int PIECES = MT * SK / 8;
    const int k0 = stage * SK;
#pragma unroll
    for (int it = 0; it < (PIECES + 255) / 256; ++it) {
      const int piece = it * 256 + tid;
      if (piece < PIECES) {
        const int r = piece / (SK / 8), kk = (piece % (SK / 8)) * 8;
        const int src = s_rows[r];
        uint4 v = make_uint4(0, 0, 0, 0);
        if (src >= 0 && k0 + kk < a.K)
          v = *reinterpret_cast<const uint4*>(a.X + static_cast<int64_t>(src) * a.K + k0 + kk);
        *reinterpret_cast<uint4*>(&s_x[buf][r * XS + kk]) = v;
      }
    }
  };

  f32x4_v acc[RT][TB];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[rt][tb] = f32x4_v{0.f, 0.f, 0.f, 0.f};

  const int tb_used = (m_count + 15) / 16;
  load_w(0);
  for (int s = 0; s < nstages; ++s) {
    const int buf = s & 1;
    stage_x(s, buf);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      // widen chunk j, then refill its ring slot with chunk j of stage s + 1
      bf16x8_v wa[RT][2];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) wr[j][rt].get(wa[rt][0], wa[rt][1]);
      if (s + 1 < nstages) {
        const int c = (s + 1) * KS + j;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          if (c < nchunks && wrow[rt] < a.N)
            wr[j][rt].load(Wg + static_cast<int64_t>(wrow[rt]) * a.K + c * 64 + g4 * 16);
          else
            wr[j][rt].zero();
        }
      }
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        if (tb < tb_used) {
          const bf16_t* xp = &s_x[buf][(tb * 16 + l16) * XS + j * 64 + g4 * 16];
          const bf16x8_v x0 = *reinterpret_cast<const bf16x8_v*>(xp);
          const bf16x8_v x1 = *reinterpret_cast<const bf16x8_v*>(xp + 8);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            acc[rt][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[rt][0], x0, acc[rt][tb], 0, 0, 0);
            acc[rt][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[rt][1], x1, acc[rt][tb], 0, 0, 0);
          }
        }
      }
    }
  }

  // ---- epilogue: lane holds rows 4 g4 + r of each 16-row tile, token l16
  const float* sc = a.w_scale ? a.w_scale + static_cast<int64_t>(grp) * a.s_group_stride : nullptr;
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int t = tb * 16 + l16;
    if (t >= m_count) continue;
    const int dst = s_dst[t];
    if (MODE == kGateUp) {
      const int I = a.N / 2;
      const int n = tx * 64 + wave * 16 + g4 * 4;
      if (n >= I) continue;
      float hv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float sg = sc ? sc[n + r] : 1.f, su = sc ? sc[I + n + r] : 1.f;
        hv[r] = gelu_erf(acc[0][tb][r] * sg) * (acc[1][tb][r] * su);
      }
      uint2 pk;
      pk.x = pack_bf16x2(hv[0], hv[1]);
      pk.y = pack_bf16x2(hv[2], hv[3]);
      *reinterpret_cast<uint2*>(static_cast<bf16_t*>(a.out) + static_cast<int64_t>(dst) * I + n) = pk;
    } else {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int n = tx * (64 * RT) + wave * (16 * RT) + rt * 16 + g4 * 4;
        if (n >= a.N) continue;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = acc[rt][tb][r] * (sc ? sc[n + r] : 1.f);
        if (MODE == kDown) {
          const float g = a.gates[dst];
          float* o = static_cast<float*>(a.out) + static_cast<int64_t>(dst) * a.N + n;
          *reinterpret_cast<float4*>(o) = make_float4(g * v[0], g * v[1], g * v[2], g * v[3]);
        } else if (a.out_dtype == DG_F32) {
          float* o = static_cast<float*>(a.out) + static_cast<int64_t>(dst) * a.N + n;
          if (a.accumulate) {
            float4 c = *reinterpret_cast<float4*>(o);
            *reinterpret_cast<float4*>(o) = make_float4(c.x + v[0], c.y + v[1], c.z + v[2], c.w + v[3]);
          } else {
            *reinterpret_cast<float4*>(o) = make_float4(v[0], v[1], v[2], v[3]);
          }
        } else {
          bf16_t* o = static_cast<bf16_t*>(a.out) + static_cast<int64_t>(dst) * a.N + n;
          uint2 pk;
          pk.x = pack_bf16x2(v[0], v[1]);
          pk.y = pack_bf16x2(v[2], v[3]);
          *reinterpret_cast<uint2*>(o) = pk;
        }
      }
    }
  }
}

}  // namespace dg
