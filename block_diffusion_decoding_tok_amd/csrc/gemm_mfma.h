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
// the same k order, so the products pair up.  The weight ring holds PF
// stages, so weight loads are issued PF stages before their use.  fp8 (OCP e4m3fn) weights are
// widened to bf16 exactly in registers; their per-row scale is applied in the
// epilogue, where it factors out of the sum.
//
// Modes:
//   kGateUp  rows of tile 0 = gate rows n0 + 16 wave + i, tile 1 = up rows
//            I + n0 + ...; epilogue h = GELU_erf(s_g acc0) * (s_u acc1) -> bf16
//            h[sorted position, n]; tokens are the slots of one expert.
//   kDown    A rows = W_down rows; X = h rows in sorted order; epilogue
//            y_slot[slot, row] = gate[slot] * s * acc (bf16).
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
  // tiled 16 x 64 blocks (bf16 / fp8): elements between the blocks of
  // consecutive 16-row tiles and between consecutive 64-k chunks of a tile.
  // w_chunk_stride == 0: one matrix, each tile's chunks contiguous (tile
  // stride K / 64 * 1024, chunk stride 1024); a stack of experts stores the
  // chunk c of every expert's tiles together (tile stride 1024, chunk stride
  // E * N / 16 * 1024)
  int64_t w_tile_stride;
  int64_t w_chunk_stride;
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
  void* out;                // gate_up: h bf16 [T*k, I]; down: y_slot bf16 [T*k, D];
                            // dense: [M, N] in out_dtype
  int out_dtype;            // dense: DG_BF16 / DG_F32
  int accumulate;           // dense: out (f32) += result
  int n_tiles_x;            // row tiles per group
  int n_tiles_y;            // token-tile slots
  int n_tiles_total;        // logical workgroups (x * y)
  int y_fastest;            // dense: logical order with token tiles of the same rows adjacent
  int x_tiled;              // dense: X in the tiled activation layout (xtile_offset)
  // dense QKV projection with the RoPE epilogue (gemm_splitk_kernel; a
  // 128-row tile is one head of 128, a 64-row tile the row pairs (d, d + 64)
  // of d in [0, 32) or [32, 64) of one head): out is unused; q (rotated,
  // scaled by q_scale) goes to the packed attention layout, k (rotated) and v
  // to the caches
  int rope;
  const float2* rope_tab;   // (cos, sin) [M, 64] of the tokens' positions (RopeTable)
  const int32_t* prefix_len;
  int Lq, Hq, Hkv, Tmax;
  float q_scale;
  bf16_t* q_out;
  bf16_t* k_cache;
  bf16_t* v_cache;
  // step gate (step_gate_closed): null outside the adaptive block loop
  const int32_t* gate;
  int gate_n;
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

// Cache policy of the weight streams.  In the one-wave expert kernel
// (gemm_wave_kernel) the item that is its expert's last token tile loads the
// weights with the nontemporal hint, so that rows read for the last time in
// the launch do not displace what the step reuses from the caches
// (activations, routing tables, the KV cache); an expert's earlier token
// tiles load them with the default policy and leave them in L2 for the later
// ones.  Measured on the 30-layer step at 256 tokens: the hint on every item
// +2.3% against no hint, but 16% of the weight bytes fetched twice; the hint
// on last tiles only a further +1.4%; on single-tile experts only, -2%.  The
// LDS-staged expert tiles (more tokens per expert) and the dense projections
// keep the default policy: with the hint they measured 1.7% (a thousand
// tokens) and 1% slower.
constexpr bool kNtWaveW = true;
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
  const u32x4_nt t = __builtin_nontemporal_load(static_cast<const u32x4_nt*>(p));
  return make_uint4(t[0], t[1], t[2], t[3]);
}
__device__ __forceinline__ uint2 load_nt8(const void* p) {
  typedef unsigned int u32x2_nt __attribute__((ext_vector_type(2)));
  const u32x2_nt t = __builtin_nontemporal_load(static_cast<const u32x2_nt*>(p));
  return make_uint2(t[0], t[1]);
}
template <bool NT>
__device__ __forceinline__ uint4 load_w16(const void* p) {
  return NT ? load_nt16(p) : *static_cast<const uint4*>(p);
}

// Weight formats of the streamed A operand.
constexpr int kWBf16 = 0;   // bf16 values
constexpr int kWFp8 = 1;    // OCP e4m3fn bytes, per-row scale in the epilogue
constexpr int kWMx4 = 2;    // OCP MXFP4: E2M1 pairs per byte + an E8M0 scale per 32 k

template <int WF> struct WChunk;
template <> struct WChunk<kWFp8> {
  uint4 q;
  template <int SECOND = 0, bool NT = false>
  __device__ void load(const uint8_t* p) { q = load_w16<NT>(p); }
  __device__ void zero() { q = make_uint4(0, 0, 0, 0); }
  __device__ void get(bf16x8_v& a, bf16x8_v& b) const { fp8x16_to_bf16(q, a, b); }
};
template <> struct WChunk<kWBf16> {
  uint4 q0, q1;
  template <int SECOND = 8, bool NT = false>
  __device__ void load(const bf16_t* p) {
    q0 = load_w16<NT>(p);
    q1 = load_w16<NT>(p + SECOND);
  }
  __device__ void zero() { q0 = q1 = make_uint4(0, 0, 0, 0); }
  __device__ void get(bf16x8_v& a, bf16x8_v& b) const {
    a = *reinterpret_cast<const bf16x8_v*>(&q0);
    b = *reinterpret_cast<const bf16x8_v*>(&q1);
  }
};
// A lane's 16 k of MXFP4 (8 bytes, the lower k in the low nibble) and the
// E8M0 scale byte of their 32-k block.  The conversion multiplies by the
// scale 2^(e - 127) (built as the float with exponent field e), so the bf16
// values are the exact weights for scale bytes 1..254 (E2M1 has 2 significant
// bits; the quantizer keeps every product a normal bf16 or zero).
template <> struct WChunk<kWMx4> {
  uint2 q;
  uint32_t s;
  template <bool NT = false>
  __device__ void load_mx(const uint8_t* codes, const uint8_t* scale) {
    q = NT ? load_nt8(codes) : *reinterpret_cast<const uint2*>(codes);
    s = *scale;
  }
  __device__ void get(bf16x8_v& a, bf16x8_v& b) const {
    const float sc = __uint_as_float(s << 23);
    bf16x2_v p[8];
    p[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q.x, sc, 0);
    p[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q.x, sc, 1);
    p[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q.x, sc, 2);
    p[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q.x, sc, 3);
    p[4] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q.y, sc, 0);
    p[5] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q.y, sc, 1);
    p[6] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q.y, sc, 2);
    p[7] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q.y, sc, 3);
    a = bf16x8_v{p[0][0], p[0][1], p[1][0], p[1][1], p[2][0], p[2][1], p[3][0], p[3][1]};
    b = bf16x8_v{p[4][0], p[4][1], p[5][0], p[5][1], p[6][0], p[6][1], p[7][0], p[7][1]};
  }
};

// Bytes of one tiled MXFP4 block (16 rows x 64 k): 512 code bytes in lane
// order (lane r + 16 q: row r, k 16 q .. 16 q + 15) and 32 scale bytes
// (16 h + r: row r, k half h).
constexpr int kMx4Block = 544;

// Address of a lane's 16 k-values of chunk c (64 k) of a 16-row weight tile,
// row-major or tile-packed (DG_LAYOUT_TILED: the tile's chunk c is one
// contiguous block of 1024 elements in lane order).
template <typename WT, bool TILED>
struct WRow {
  const WT* base;
  int64_t cstride;
  static constexpr int kSecond = TILED ? 512 : 8;   // 2-byte types: values 8..15
  __device__ void init(const WT* Wg, int row0, int K, int lane, const GemmArgs& a) {
    if (TILED) {
      const int64_t ts = a.w_chunk_stride ? a.w_tile_stride : static_cast<int64_t>(K / 64) * 1024;
      cstride = a.w_chunk_stride ? a.w_chunk_stride : 1024;
      base = Wg + static_cast<int64_t>(row0 / 16) * ts + lane * (sizeof(WT) == 1 ? 16 : 8);
    } else {
      cstride = 64;
      base = Wg + static_cast<int64_t>(row0 + (lane & 15)) * K + (lane >> 4) * 16;
    }
  }
  __device__ const WT* at(int c) const { return base + c * cstride; }
};

template <int RT, int TB, int KS, int PF, int WF, int MODE, bool TILED, int MINWG = 1>
__global__ __launch_bounds__(256, MINWG) void gemm_stream_kernel(GemmArgs a) {
  static_assert(WF != kWMx4 || TILED, "MXFP4 weights are always tile-packed");
  if (step_gate_closed(a.gate, a.gate_n)) return;
  using WT = typename std::conditional<WF == kWBf16, bf16_t, uint8_t>::type;
  constexpr int MT = 16 * TB;           // tokens per tile
  constexpr int SK = 64 * KS;           // k per LDS stage
  constexpr int XS = SK + 8;            // LDS row stride (elements)
  __shared__ __attribute__((aligned(16))) bf16_t s_x[2][MT * XS];
  __shared__ int s_rows[MT];            // source row of each token of the tile
  __shared__ int s_dst[MT];             // destination row (grouped modes)
  __shared__ int s_scan[256];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;

  // ---- row tile within the group (tx), token tile (ty), and which group /
  // token range the tile covers
  int tx = 0, ty = 0;
  int grp = 0, m0 = 0, m_count = 0, base_pos = 0;
  if (MODE == kDense) {
    const int logical = xcd_logical_tile(blockIdx.x, gridDim.x);
    if (logical >= a.n_tiles_total) return;
    tx = a.y_fastest ? logical / a.n_tiles_y : logical % a.n_tiles_x;
    ty = a.y_fastest ? logical % a.n_tiles_y : logical / a.n_tiles_x;
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
    // the grid is an upper bound of the item count: the live items are dealt
    // out evenly over the 8 XCDs (workgroup i runs on XCD i % 8) in
    // contiguous ranges with the row tiles of a token tile adjacent, so that
    // a token tile's rows are fetched into one L2 once (at a thousand tokens
    // the gathered rows outgrow an L2) and an expert's consecutive token
    // tiles still share its weight rows there
    const int n_tiles = s_scan[E - 1];
    const int live = n_tiles * a.n_tiles_x;
    const int per_xcd = (live + 7) / 8;
    const int slot = blockIdx.x / 8;
    if (slot >= per_xcd) return;
    const int item = (blockIdx.x % 8) * per_xcd + slot;
    if (item >= live) return;
    tx = item % a.n_tiles_x;
    ty = item / a.n_tiles_x;
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

  // ---- what the expert epilogue reads besides the accumulators, fetched
  // now so that its latency is not added after the last stage (the scale and
  // gate reads there each waited on the spot): the item's 128 per-row fp8
  // scales by direct-to-LDS copies (gate/up: 64 gate rows, then the 64 up
  // rows; down: 64 RT rows) and, for down, the gate of each token row
  const float* sc = a.w_scale ? a.w_scale + static_cast<int64_t>(grp) * a.s_group_stride : nullptr;
  __shared__ float s_esc[128];
  __shared__ float s_egt[MT];
  if constexpr (MODE != kDense) {
    static_assert(MODE == kGateUp || 64 * RT == 128, "128 scale rows per item");
    static_assert(MT == 64, "one wave copies the token rows' gates");
    if (sc) {
      if (wave < 2) {
        const int q = wave * 64 + lane;
        const int row = (MODE == kGateUp) ? (q < 64 ? tx * 64 + q : a.N / 2 + tx * 64 + q - 64)
                                          : tx * 128 + q;
        __builtin_amdgcn_global_load_lds(sc + row, s_esc + wave * 64, 4, 0, 0);
      }
    } else if (tid < 128) {
      s_esc[tid] = 1.f;                      // unscaled weights
    }
  }
  // down: the gate of token row tid (every thread loads one, unconditionally;
  // written to LDS by the first MT threads in the epilogue)
  float e_gt = 0.f;
  if constexpr (MODE == kDown) e_gt = a.gates[max(s_dst[min(tid, MT - 1)], 0)];

  // ---- weight rows of this wave
  const WT* Wg = static_cast<const WT*>(a.W) + static_cast<int64_t>(grp) * a.w_group_stride;
  WRow<WT, TILED> wr_at[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row0 = (MODE == kGateUp) ? (rt == 0 ? 0 : a.N / 2) + tx * 64 + wave * 16
                                       : tx * (64 * RT) + wave * (16 * RT) + rt * 16;
    wr_at[rt].init(Wg, row0, a.K, lane, a);
  }
  // MXFP4: tile blocks of 544 bytes (a tile's chunks contiguous); the lane's
  // 8 code bytes at 8 lane, the scale of its 32-k half at 512 + 16 (g4 / 2) + r
  const uint8_t* mx_codes[RT];
  const uint8_t* mx_scale[RT];
  if constexpr (WF == kWMx4) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int row0 = (MODE == kGateUp) ? (rt == 0 ? 0 : a.N / 2) + tx * 64 + wave * 16
                                         : tx * (64 * RT) + wave * (16 * RT) + rt * 16;
      const uint8_t* tile = reinterpret_cast<const uint8_t*>(Wg) +
                            static_cast<int64_t>(row0 / 16) * (a.K / 64) * kMx4Block;
      mx_codes[rt] = tile + lane * 8;
      mx_scale[rt] = tile + 512 + 16 * (g4 >> 1) + l16;
    }
  }
  auto load_chunk = [&](WChunk<WF>& w, int rt, int c) {
    if constexpr (WF == kWMx4)
      w.load_mx(mx_codes[rt] + c * kMx4Block, mx_scale[rt] + c * kMx4Block);
    else
      w.template load<WRow<WT, TILED>::kSecond>(wr_at[rt].at(c));
  };
  const int nchunks = (a.K + 63) / 64;
  const int nstages = (nchunks + KS - 1) / KS;

  // weight ring: PF stages of KS chunks in flight per wave
  WChunk<WF> wr[PF][KS][RT];
  // unconditional loads (clamped chunk; rows are in range by contract) keep
  // the compiler's memory-counter waits precise
  auto load_w = [&](int stage, WChunk<WF> (&slot)[KS][RT]) {
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      const int c = min(stage * KS + j, nchunks - 1);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) load_chunk(slot[j][rt], rt, c);
    }
  };
  // token rows: a stage of MT rows x SK k of bf16 = PIECES 16-byte pieces,
  // loaded into registers one stage ahead and written to LDS at stage start
  constexpr int PIECES = MT * SK / 8;
  constexpr int XP = (PIECES + 255) / 256;
  uint4 xr[PF][XP];                     // PF stages of token rows in flight
  // raw loads from clamped addresses; the mask is applied when the stage is
  // written to LDS (a select right after a load would wait for it at once)
  auto load_x = [&](int stage, uint4 (&slot)[XP]) {
    const int k0 = min(stage, nstages - 1) * SK;
#pragma unroll
    for (int it = 0; it < XP; ++it) {
      const int piece = it * 256 + tid;
      const int r = min(piece / (SK / 8), MT - 1), kk = (piece % (SK / 8)) * 8;
      const int src = s_rows[r];
      const int kc = min(k0 + kk, a.K - 8);
      slot[it] = *reinterpret_cast<const uint4*>(a.X + static_cast<int64_t>(src >= 0 ? src : s_rows[0]) * a.K + kc);
    }
  };
  auto store_x = [&](int stage, int buf, const uint4 (&slot)[XP]) {
    const int k0 = stage * SK;
#pragma unroll
    for (int it = 0; it < XP; ++it) {
      const int piece = it * 256 + tid;
      if (piece < PIECES) {
        const int r = piece / (SK / 8), kk = (piece % (SK / 8)) * 8;
        const bool ok = s_rows[r] >= 0 && k0 + kk < a.K;
        *reinterpret_cast<uint4*>(&s_x[buf][r * XS + kk]) = ok ? slot[it] : make_uint4(0, 0, 0, 0);
      }
    }
  };

  f32x4_v acc[RT][TB];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[rt][tb] = f32x4_v{0.f, 0.f, 0.f, 0.f};

  const int tb_used = (m_count + 15) / 16;
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    load_w(p, wr[p]);
    load_x(p, xr[p]);
  }
  for (int s0 = 0; s0 < nstages; s0 += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int s = s0 + p;
      if (s >= nstages) break;
      const int buf = s & 1;
      store_x(s, buf, xr[p]);
      __syncthreads();
      // (one stage in flight: no refill past the last stage, whose loads the
      // epilogue would otherwise wait for)
      const bool refill = PF > 1 || s + PF < nstages;
      if (refill) load_x(s + PF, xr[p]);
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        // widen chunk j of stage s, then refill its slot with stage s + PF
        bf16x8_v wa[RT][2];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) wr[p][j][rt].get(wa[rt][0], wa[rt][1]);
        const int c = min((s + PF) * KS + j, nchunks - 1);
        if (refill) {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) load_chunk(wr[p][j][rt], rt, c);
        }
        if (s * KS + j >= nchunks) continue;
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
  }

  // ---- epilogue: lane holds rows 4 g4 + r of each 16-row tile, token l16
  if constexpr (MODE != kDense) {
    // expert modes: the workgroup's MT rows x NC columns go through LDS (the
    // token stages are free once every wave is past the last one), so that
    // each destination row leaves as one run of 16-byte pieces
    constexpr int NC = MODE == kGateUp ? 64 : 64 * RT;
    constexpr int OS = NC + 8;
    static_assert(MT * OS <= 2 * MT * XS, "output tile fits the token stages");
    bf16_t* s_o = &s_x[0][0];
    // the copies issued at the start (each wave waits for its own; the
    // barrier then makes them visible to all)
    if (MODE == kDown && tid < MT) s_egt[tid] = e_gt;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int t = tb * 16 + l16;
      if (MODE == kGateUp) {
        const int q = wave * 16 + g4 * 4;     // item row of gate column tx 64 + q
        float hv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          hv[r] = gelu_erf(acc[0][tb][r] * s_esc[q + r]) * (acc[1][tb][r] * s_esc[64 + q + r]);
        uint2 pk;
        pk.x = pack_bf16x2(hv[0], hv[1]);
        pk.y = pack_bf16x2(hv[2], hv[3]);
        *reinterpret_cast<uint2*>(&s_o[t * OS + wave * 16 + g4 * 4]) = pk;
      } else {
        const float g = t < m_count ? s_egt[t] : 0.f;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const int nl = wave * (16 * RT) + rt * 16 + g4 * 4;
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = g * acc[rt][tb][r] * s_esc[nl + r];
          uint2 pk;
          pk.x = pack_bf16x2(v[0], v[1]);
          pk.y = pack_bf16x2(v[2], v[3]);
          *reinterpret_cast<uint2*>(&s_o[t * OS + nl]) = pk;
        }
      }
    }
    __syncthreads();
    constexpr int PR = NC / 8;               // 16-byte pieces per row
    const int ld = MODE == kGateUp ? a.N / 2 : a.N;
#pragma unroll
    for (int it = 0; it < (MT * PR + 255) / 256; ++it) {
      const int q = it * 256 + tid;
      const int row = q / PR, c8 = q % PR;
      if (q < MT * PR && row < m_count)
        *reinterpret_cast<uint4*>(static_cast<bf16_t*>(a.out) + static_cast<int64_t>(s_dst[row]) * ld +
                                  tx * NC + c8 * 8) =
            *reinterpret_cast<const uint4*>(&s_o[row * OS + c8 * 8]);
    }
    return;
  }
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
          bf16_t* o = static_cast<bf16_t*>(a.out) + static_cast<int64_t>(dst) * a.N + n;
          uint2 pk;
          pk.x = pack_bf16x2(g * v[0], g * v[1]);
          pk.y = pack_bf16x2(g * v[2], g * v[3]);
          *reinterpret_cast<uint2*>(o) = pk;
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


namespace dg {

// One-wave workgroups for the grouped (expert) GEMMs at canvas-sized token
// counts.  A work item is (token tile of 16 * TB rows of one expert, group of
// RT weight tiles of 16 rows): for gate/up, RT/2 gate tiles and the matching
// RT/2 up tiles (8 * RT intermediate columns); for down, 16 * RT output rows.
// Every item streams the same weight bytes, and a tile holds up to 16 * TB
// tokens so that the few experts that draw many tokens need few items: the
// launch then fits (nearly) one round of resident waves instead of ending
// with a short extra round.  Token blocks of a tile past the expert's count
// skip their MFMAs (wave-uniform).  The item decode runs in registers with
// wave shuffles.  The K loop streams a ring of NR chunks of both operands,
// unconditional loads in a pinned order; no LDS, no barrier.  (Giving a wave
// all of an expert's tokens in consecutive passes measured slower: the busy
// experts' items then take several times longer than the rest.)
constexpr bool kWaveIssueFirst = false;

template <int RT, int TB, int NR, int WF, int MODE, bool TILED, int WPE = 1>
__global__ __launch_bounds__(64, WPE) void gemm_wave_kernel(GemmArgs a) {
  static_assert(MODE == kGateUp || MODE == kDown, "grouped modes only");
  static_assert(MODE != kGateUp || RT % 2 == 0, "gate/up needs paired tiles");
  static_assert(WF != kWMx4 || TILED, "MXFP4 weights are always tile-packed");
  using WT = typename std::conditional<WF == kWBf16, bf16_t, uint8_t>::type;
  constexpr int MT = 16 * TB;
  if (step_gate_closed(a.gate, a.gate_n)) return;
  const int lane = threadIdx.x;
  const int l16 = lane & 15, g4 = lane >> 4;

  // ---- item decode: inclusive scan of MT-token tiles per expert (E <= 256)
  const int E = a.n_groups;
  int cnt[4], incl[4];
  int carry = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = q * 64 + lane;
    cnt[q] = e < E ? (a.offsets[e + 1] - a.offsets[e] + MT - 1) / MT : 0;
    int v = cnt[q];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(v, o);
      if (lane >= o) v += t;
    }
    incl[q] = v + carry;
    carry += __shfl(v, 63);
  }
  // The grid is an upper bound of the item count; the carry * n_tiles_x
  // live items are dealt out evenly over the 8 XCDs (workgroup i runs on XCD
  // i % 8), each XCD taking a contiguous range in which the token tiles of a
  // row group are adjacent, so an expert's tiles share its weight rows in
  // one L2.
  const int live = carry * a.n_tiles_x;
  const int per_xcd = (live + 7) / 8;
  const int slot = blockIdx.x / 8;
  if (slot >= per_xcd) return;
  const int item = (blockIdx.x % 8) * per_xcd + slot;
  if (item >= live) return;
  const int tx = item / carry, ty = item % carry;
  int grp = -1, first_tile = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint64_t m = __ballot(incl[q] > ty);
    if (grp < 0 && m) {
      const int src_lane = __ffsll(static_cast<unsigned long long>(m)) - 1;
      grp = q * 64 + src_lane;
      first_tile = __shfl(incl[q] - cnt[q], src_lane);
    }
  }
  // wave-uniform from here on: keep the expert and tile bases in SGPRs
  grp = __builtin_amdgcn_readfirstlane(grp);
  first_tile = __builtin_amdgcn_readfirstlane(first_tile);
  const int base_pos = a.offsets[grp];
  const int m0 = (ty - first_tile) * MT;
  const int m_count = min(MT, a.offsets[grp + 1] - base_pos - m0);
  const int tb_used = (m_count + 15) / 16;   // wave-uniform
  bool xok[TB];
  int p_pos[TB];
  const bf16_t* xp[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int m = tb * 16 + l16;
    xok[tb] = m < m_count;
    p_pos[tb] = base_pos + m0 + (xok[tb] ? m : 0);
    const int src = (MODE == kGateUp) ? a.sorted_rows[p_pos[tb]] / a.topk : p_pos[tb];
    xp[tb] = a.X + static_cast<int64_t>(src) * a.K + g4 * 16;
  }

  // weight tiles: uniform tile bases + one per-lane offset (TILED: the
  // lane's 16 values of chunk c at c * 1024 + 16 (or 8) * lane elements;
  // MXFP4: codes at c * 544 + 8 * lane bytes, the scale of its 32-k half at
  // c * 544 + 512 + 16 (q / 2) + r; row-major: row lane % 16, k 16 (lane / 16)
  // + 64 c)
  const WT* Wg = static_cast<const WT*>(a.W) + static_cast<int64_t>(grp) * a.w_group_stride;
  // elements between a tile's consecutive 64-k chunks, and between tiles
  const int64_t kChunk = WF == kWMx4 ? kMx4Block
                         : TILED     ? (a.w_chunk_stride ? a.w_chunk_stride : 1024)
                                     : 64;
  const int64_t tile_stride = WF == kWMx4 ? static_cast<int64_t>(a.K / 64) * kMx4Block
                              : (a.w_chunk_stride ? a.w_tile_stride : static_cast<int64_t>(a.K / 64) * 1024);
  const WT* wtile[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row0 = (MODE == kGateUp)
                         ? (rt < RT / 2 ? 0 : a.N / 2) + tx * (8 * RT) + (rt % (RT / 2)) * 16
                         : tx * (16 * RT) + rt * 16;
    wtile[rt] = TILED ? Wg + static_cast<int64_t>(row0 / 16) * tile_stride
                      : Wg + static_cast<int64_t>(row0) * a.K;
  }
  const int w_lane = WF == kWMx4 ? lane * 8
                     : TILED     ? lane * (sizeof(WT) == 1 ? 16 : 8)
                                 : (lane & 15) * a.K + (lane >> 4) * 16;
  const int s_lane = 512 + 16 * (g4 >> 1) + l16;   // MXFP4 only
  const int nchunks = a.K / 64;

  struct Slot {
    uint4 x[TB][2];
    WChunk<WF> w[RT];
  };
  // cache policy of this item's weight loads (wave-uniform): the hint on
  // the expert's last token tile only
  const int grp_tiles = (a.offsets[grp + 1] - base_pos + MT - 1) / MT;
  const bool item_nt = kNtWaveW && ty - first_tile == grp_tiles - 1;

  // With one chunk in flight (NR = 1), what the epilogue reads besides the
  // accumulators is fetched before the weight stream, so that its latency is
  // not added after the last chunk (the scale reads there each waited on the
  // spot): the item's per-row fp8 scales (16 RT rows; gate/up: the 8 RT gate
  // rows, then the 8 RT up rows) copied into LDS (direct-to-LDS, no
  // registers held), and for down each token row's slot and gate (canvas
  // step +2.8%; the deeper-ring items of a few tokens measured slower with
  // it and read them at the end).
  constexpr bool kEpiPrefetch = NR == 1;
  const float* sc = a.w_scale ? a.w_scale + static_cast<int64_t>(grp) * a.s_group_stride : nullptr;
  constexpr int kScRows = 16 * RT;
  constexpr int kScPad = (kScRows + 63) / 64 * 64;   // whole 64-lane copies
  __shared__ float s_sc[kEpiPrefetch ? kScPad : 1];
  if constexpr (kEpiPrefetch) {
    if (!sc) {
#pragma unroll
      for (int it = 0; it < kScPad / 64; ++it) s_sc[it * 64 + lane] = 1.f;   // unscaled weights
    } else {
#pragma unroll
      for (int it = 0; it < kScPad / 64; ++it) {
        const int q = min(it * 64 + lane, kScRows - 1);   // lanes past the rows repeat the last
        const int row = (MODE == kGateUp) ? (q < 8 * RT ? tx * (8 * RT) + q : a.N / 2 + tx * (8 * RT) + q - 8 * RT)
                                          : tx * (16 * RT) + q;
        __builtin_amdgcn_global_load_lds(sc + row, s_sc + it * 64, 4, 0, 0);
      }
    }
  }
  int e_slot[TB];
  float e_gate[TB];
  if constexpr (MODE == kDown && kEpiPrefetch) {
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) e_slot[tb] = xok[tb] ? a.sorted_rows[p_pos[tb]] : -1;
  }
  const uint4 zero4 = make_uint4(0, 0, 0, 0);
  f32x4_v acc[RT][TB];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[rt][tb] = f32x4_v{0.f, 0.f, 0.f, 0.f};
  auto stream_k = [&](auto nt_tag) {
    constexpr bool NT = decltype(nt_tag)::value;
    Slot ring[NR];
    auto issue = [&](Slot& sl, int c) {
      const int cc = min(c, nchunks - 1);
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        sl.x[tb][0] = *reinterpret_cast<const uint4*>(xp[tb] + cc * 64);
        sl.x[tb][1] = *reinterpret_cast<const uint4*>(xp[tb] + cc * 64 + 8);
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        if constexpr (WF == kWMx4)
          sl.w[rt].template load_mx<NT>(wtile[rt] + w_lane + cc * kChunk,
                                        wtile[rt] + s_lane + cc * kChunk);
        else
          sl.w[rt].template load<WRow<WT, TILED>::kSecond, NT>(wtile[rt] + w_lane + cc * kChunk);
      }
    };
#pragma unroll
    for (int p = 0; p < NR; ++p) {
      issue(ring[p], p);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (MODE == kDown && kEpiPrefetch) {
      // the gates of the item's slots, behind the first weight chunks
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) e_gate[tb] = e_slot[tb] >= 0 ? a.gates[e_slot[tb]] : 0.f;
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int c0 = 0; c0 < nchunks; c0 += NR) {
#pragma unroll
      for (int p = 0; p < NR; ++p) {
        // kWaveIssueFirst: refill the slot before its MMAs (one more slot of
        // registers, loads issued one compute step earlier); otherwise refill
        // it right after
        const Slot cur = ring[p];
        if (kWaveIssueFirst) {
          __builtin_amdgcn_sched_barrier(0);
          issue(ring[p], c0 + p + NR);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (c0 + p < nchunks) {
          bf16x8_v xa[TB][2];
#pragma unroll
          for (int tb = 0; tb < TB; ++tb) {
            const uint4 u0 = xok[tb] ? cur.x[tb][0] : zero4;
            const uint4 u1 = xok[tb] ? cur.x[tb][1] : zero4;
            xa[tb][0] = *reinterpret_cast<const bf16x8_v*>(&u0);
            xa[tb][1] = *reinterpret_cast<const bf16x8_v*>(&u1);
          }
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            bf16x8_v w0, w1;
            cur.w[rt].get(w0, w1);
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
              if (tb == 0 || tb < tb_used) {
                acc[rt][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w0, xa[tb][0], acc[rt][tb], 0, 0, 0);
                acc[rt][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w1, xa[tb][1], acc[rt][tb], 0, 0, 0);
              }
            }
          }
        }
        // (one chunk in flight: no refill past the last chunk, whose load
        // the epilogue would otherwise wait for before reusing its registers)
        if (!kWaveIssueFirst && (NR > 1 || c0 + p + NR < nchunks)) {
          __builtin_amdgcn_sched_barrier(0);
          issue(ring[p], c0 + p + NR);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };
  if (item_nt)
    stream_k(std::integral_constant<bool, true>{});
  else
    stream_k(std::integral_constant<bool, false>{});

  // ---- epilogue (lane: rows 4 g4 + r of each 16-row tile, token l16 of
  // each 16-token block).  With the prefetch, the scale copies into LDS are
  // the only loads still in flight (no refill was issued past the last chunk).
  if (kEpiPrefetch && sc) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  // scale of item row q (the epilogue's only use of sc)
  auto row_scale = [&](int q) {
    if constexpr (kEpiPrefetch) return s_sc[q];
    const int row = (MODE == kGateUp) ? (q < 8 * RT ? tx * (8 * RT) + q : a.N / 2 + tx * (8 * RT) + q - 8 * RT)
                                      : tx * (16 * RT) + q;
    return sc ? sc[row] : 1.f;
  };
  if constexpr (MODE == kGateUp) {
    // h = GELU(gate) * up for the item's 16 TB sorted positions (consecutive
    // rows of h) x 8 RT columns, staged through LDS like the down epilogue
    // below so that each row leaves as one run of 16 RT bytes
    const int I = a.N / 2;
    constexpr int NC = 8 * RT;               // columns of the item
    constexpr int HS = NC + 8;               // LDS row stride (elements)
    __shared__ __attribute__((aligned(16))) bf16_t s_h[16 * TB * HS];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int row = tb * 16 + l16;
#pragma unroll
      for (int i = 0; i < RT / 2; ++i) {
        float hv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          // item row of gate column tx NC + q (its up row: q + 8 RT)
          const int q = i * 16 + g4 * 4 + r;
          const float sg = row_scale(q), su = row_scale(8 * RT + q);
          hv[r] = gelu_erf(acc[i][tb][r] * sg) * (acc[RT / 2 + i][tb][r] * su);
        }
        uint2 pk;
        pk.x = pack_bf16x2(hv[0], hv[1]);
        pk.y = pack_bf16x2(hv[2], hv[3]);
        *reinterpret_cast<uint2*>(&s_h[row * HS + i * 16 + g4 * 4]) = pk;
      }
    }
    __syncthreads();                         // one wave: orders the LDS writes and reads
    constexpr int PR = NC / 8;               // 16-byte pieces per row
    constexpr int PIECES = 16 * TB * PR;
#pragma unroll
    for (int it = 0; it < (PIECES + 63) / 64; ++it) {
      const int q = it * 64 + lane;
      const int row = q / PR, c8 = q % PR;
      if (q < PIECES && row < m_count) {
        const uint4 v = *reinterpret_cast<const uint4*>(&s_h[row * HS + c8 * 8]);
        *reinterpret_cast<uint4*>(static_cast<bf16_t*>(a.out) +
                                  static_cast<int64_t>(base_pos + m0 + row) * I + tx * NC + c8 * 8) = v;
      }
    }
  }
  if constexpr (MODE == kDown) {
    // The item's 16 TB slot rows x 16 RT columns go through LDS, so that the
    // stores leave as runs of 32 RT bytes per slot row (16 bytes per lane)
    // instead of 8-byte pieces: first each lane puts its gate- and
    // scale-weighted values of token l16 (rows 4 g4 .. 4 g4 + 3 of every
    // tile) into row tb * 16 + l16; then lane l copies 16-byte pieces.
    constexpr int NC = 16 * RT;              // columns of the item
    constexpr int YS = NC + 8;               // LDS row stride (elements)
    __shared__ __attribute__((aligned(16))) bf16_t s_y[16 * TB * YS];
    __shared__ int s_slot[16 * TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int row = tb * 16 + l16;
      int slot;
      float g;
      if constexpr (kEpiPrefetch) {
        slot = e_slot[tb];
        g = e_gate[tb];
      } else {
        slot = xok[tb] ? a.sorted_rows[p_pos[tb]] : -1;
        g = xok[tb] ? a.gates[slot] : 0.f;
      }
      if (g4 == 0) s_slot[row] = slot;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = g * acc[rt][tb][r] * row_scale(rt * 16 + g4 * 4 + r);
        uint2 pk;
        pk.x = pack_bf16x2(v[0], v[1]);
        pk.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2*>(&s_y[row * YS + rt * 16 + g4 * 4]) = pk;
      }
    }
    __syncthreads();                         // one wave: orders the LDS writes and reads
    constexpr int PR = NC / 8;               // 16-byte pieces per row
    constexpr int PIECES = 16 * TB * PR;
#pragma unroll
    for (int it = 0; it < (PIECES + 63) / 64; ++it) {
      const int q = it * 64 + lane;
      if (q < PIECES) {
        const int row = q / PR, c8 = q % PR;
        const int slot = s_slot[row];
        const uint4 v = *reinterpret_cast<const uint4*>(&s_y[row * YS + c8 * 8]);
        if (slot >= 0)
          *reinterpret_cast<uint4*>(static_cast<bf16_t*>(a.out) + static_cast<int64_t>(slot) * a.N +
                                    tx * NC + c8 * 8) = v;
      }
    }
  }
}

}  // namespace dg

namespace dg {

// Dense GEMM for canvas-sized token counts (M <= 1024), bf16 weights:
// out[m, n] = sum_k X[m, k] W[n, k].  A workgroup owns a tile of 16 * RT
// weight rows x 16 * TB tokens; its NW waves split the K / 64 chunks into NW
// contiguous ranges (K % 64 == 0), so a projection with few output tiles
// still fills the chip, and each wave streams its weight rows and token rows
// through a register ring of NR chunks (unconditional loads, pinned issue
// order).  The NW partial accumulators are summed through LDS in wave order
// (fixed order: deterministic), one thread per (row tile, token block, lane)
// quad of outputs.
// Refill a ring slot before its MMAs (one more slot of registers, loads one
// compute step earlier) or right after them.
constexpr bool kSplitIssueFirst = false;

template <int RT, int TB, int NR, int NW, bool TILED, int WPE = 1>
__global__ __launch_bounds__(64 * NW, WPE) void gemm_splitk_kernel(GemmArgs a) {
  static_assert(RT * TB * 64 <= 64 * NW * 4, "at most four output quads per thread");
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  __shared__ __attribute__((aligned(16))) float s_acc[4][RT * TB * 4][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int logical = xcd_logical_tile(blockIdx.x, gridDim.x);
  if (logical >= a.n_tiles_total || step_gate_closed(a.gate, a.gate_n)) return;
  constexpr bool kRopeTile = RT == 8 || RT == 4 || RT == 2;
  const int tx = logical / a.n_tiles_y;       // row tile (token tiles adjacent)
  const int ty = logical % a.n_tiles_y;
  const int m0 = ty * 16 * TB;
  const int n0 = tx * 16 * RT;
  const int nch_all = a.K / 64;
  const int c_begin = wave * nch_all / NW;
  const int nchunks = (wave + 1) * nch_all / NW - c_begin;   // >= 1 when K >= 64 * NW
  // 16-row tile of the weights behind accumulator row tile rt: consecutive,
  // except RoPE tiles of 64 rows, which take row tiles {0, 1, 4, 5} or
  // {2, 3, 6, 7} of head tx / 2, and of 32 rows, row tiles {j, j + 4} of head
  // tx / 4 (j = tx % 4), so that both rows of every rotated pair are here
  auto row16 = [&](int rt) {
    if (RT == 4 && a.rope) return (tx >> 1) * 8 + (tx & 1) * 2 + (rt & 1) + (rt >> 1) * 4;
    if (RT == 2 && a.rope) return (tx >> 2) * 8 + (tx & 3) + rt * 4;
    return n0 / 16 + rt;
  };

  // uniform tile bases (SGPRs) + one per-lane offset, as in gemm_wave_kernel
  const bf16_t* W = static_cast<const bf16_t*>(a.W);
  const bf16_t* wtile[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
    wtile[rt] = TILED ? W + static_cast<int64_t>(row16(rt)) * (a.K / 64) * 1024
                      : W + static_cast<int64_t>(row16(rt)) * 16 * a.K;
  const int w_lane = TILED ? lane * 8 : (lane & 15) * a.K + (lane >> 4) * 16;
  constexpr int kChunk = TILED ? 1024 : 64;
  // activations: row-major (16 token rows x 16 bytes per load) or tiled (one
  // 1 KB block per load; token blocks past the last one are clamped to it,
  // their rows masked below)
  const int x_chunk = a.x_tiled ? 1024 : 64, x_second = a.x_tiled ? 512 : 8;
  const bf16_t* xp[TB];
  bool xok[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int m = m0 + tb * 16 + l16;
    xok[tb] = m < a.M;
    if (a.x_tiled) {
      const int blk = min(m0 / 16 + tb, (a.M + 15) / 16 - 1);
      xp[tb] = a.X + (static_cast<int64_t>(blk) * (a.K / 64) + c_begin) * 1024 + lane * 8;
    } else {
      xp[tb] = a.X + static_cast<int64_t>(xok[tb] ? m : m0) * a.K + c_begin * 64 + g4 * 16;
    }
  }

  struct Slot {
    uint4 x[TB][2];
    uint4 w[RT][2];
  };
  Slot ring[NR];
  auto issue = [&](Slot& sl, int c) {
    const int cc = min(c, nchunks - 1);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const bf16_t* pw = wtile[rt] + w_lane + (c_begin + cc) * kChunk;
      sl.w[rt][0] = *reinterpret_cast<const uint4*>(pw);
      sl.w[rt][1] = *reinterpret_cast<const uint4*>(pw + WRow<bf16_t, TILED>::kSecond);
    }
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      sl.x[tb][0] = *reinterpret_cast<const uint4*>(xp[tb] + cc * x_chunk);
      sl.x[tb][1] = *reinterpret_cast<const uint4*>(xp[tb] + cc * x_chunk + x_second);
    }
  };
  const uint4 zero4 = make_uint4(0, 0, 0, 0);
  f32x4_v acc[RT][TB];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[rt][tb] = f32x4_v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < NR; ++p) {
    issue(ring[p], p);
    __builtin_amdgcn_sched_barrier(0);
  }
  // one chunk step: the MMAs of chunk c from ring slot p; with `refill` the
  // slot is then loaded with chunk c + NR (before the MMAs under
  // kSplitIssueFirst)
  auto step = [&](int p, int c, bool refill) {
    const Slot cur = ring[p];
    if (kSplitIssueFirst && refill) {
      __builtin_amdgcn_sched_barrier(0);
      issue(ring[p], c + NR);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (c < nchunks) {
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const uint4 u0 = xok[tb] ? cur.x[tb][0] : zero4, u1 = xok[tb] ? cur.x[tb][1] : zero4;
        const bf16x8_v x0 = *reinterpret_cast<const bf16x8_v*>(&u0);
        const bf16x8_v x1 = *reinterpret_cast<const bf16x8_v*>(&u1);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const bf16x8_v w0 = *reinterpret_cast<const bf16x8_v*>(&cur.w[rt][0]);
          const bf16x8_v w1 = *reinterpret_cast<const bf16x8_v*>(&cur.w[rt][1]);
          acc[rt][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w0, x0, acc[rt][tb], 0, 0, 0);
          acc[rt][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w1, x1, acc[rt][tb], 0, 0, 0);
        }
      }
    }
    if (!kSplitIssueFirst && refill) {
      __builtin_amdgcn_sched_barrier(0);
      issue(ring[p], c + NR);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Tiles of up to 64 weight rows: blocks whose every refill is a chunk
  // still to come, then at most two blocks that refill only while there is
  // one, so that no loads past the last chunk are in flight when the
  // epilogue's own reads (issued below, before the reduction) are waited
  // for.  Tiles of 128 rows keep one loop with clamped refills: the peeled
  // tail costs them registers they do not have.
  constexpr bool kEpiPf = RT <= 4;
  if constexpr (kEpiPf) {
    const int n_full = nchunks > NR ? (nchunks - NR) / NR * NR : 0;
    int c0 = 0;
    for (; c0 < n_full; c0 += NR) {
#pragma unroll
      for (int p = 0; p < NR; ++p) step(p, c0 + p, true);
    }
    for (; c0 < nchunks; c0 += NR) {
#pragma unroll
      for (int p = 0; p < NR; ++p) step(p, c0 + p, c0 + p + NR < nchunks);
    }
  } else {
    for (int c0 = 0; c0 < nchunks; c0 += NR) {
#pragma unroll
      for (int p = 0; p < NR; ++p) step(p, c0 + p, true);
    }
  }

  // ---- the epilogue's global reads, issued now so that they complete while
  // the partial sums pass through LDS: the RoPE form's cache length and
  // (cos, sin) of each quad's token, the accumulate form's f32 residual
  constexpr int kPairsAll = (RT / 2) * TB * 64;
  constexpr int kQuadsAll = RT * TB * 64;
  constexpr int kPfR = (kPairsAll + 64 * NW - 1) / (64 * NW);
  constexpr int kPfA = (kQuadsAll + 64 * NW - 1) / (64 * NW);
  int pf_p[kRopeTile ? kPfR : 1];
  float4 pf_cs[kRopeTile ? kPfR : 1][2];
  float4 pf_c[kPfA];
  if constexpr (kRopeTile && kEpiPf) {
    if (a.rope) {
#pragma unroll
      for (int k = 0; k < kPfR; ++k) {
        const int q = min(k * 64 * NW + tid, kPairsAll - 1);
        const int ql = q & 63, blk = q >> 6;
        const int rt = blk / TB, tb = blk % TB;
        const int m = min(m0 + tb * 16 + (ql & 15), a.M - 1);
        const int d0 = (row16(rt) % 8) * 16 + (ql >> 4) * 4;
        pf_p[k] = a.prefix_len[m / a.Lq];
        const float4* cs = reinterpret_cast<const float4*>(a.rope_tab + static_cast<int64_t>(m) * 64 + d0);
        pf_cs[k][0] = cs[0];
        pf_cs[k][1] = cs[1];
      }
    }
  }
  if (kEpiPf && a.accumulate && a.out_dtype == DG_F32 && !(kRopeTile && a.rope)) {
#pragma unroll
    for (int k = 0; k < kPfA; ++k) {
      const int q = min(k * 64 * NW + tid, kQuadsAll - 1);
      const int ql = q & 63, blk = q >> 6;
      const int rt = blk / TB, tb = blk % TB;
      const int n = n0 + rt * 16 + (ql >> 4) * 4;
      const int m = min(m0 + tb * 16 + (ql & 15), a.M - 1);
      pf_c[k] = *reinterpret_cast<const float4*>(static_cast<const float*>(a.out) + static_cast<int64_t>(m) * a.N + n);
    }
  }

  // ---- deterministic split-K reduction through LDS: with eight waves, wave
  // w + 4 hands its partial to wave w first; then the four partials are
  // summed in wave order
  if (NW == 8) {
    if (wave >= 4) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
          for (int r = 0; r < 4; ++r) s_acc[wave - 4][(rt * TB + tb) * 4 + r][lane] = acc[rt][tb][r];
    }
    __syncthreads();
    if (wave < 4) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[rt][tb][r] += s_acc[wave][(rt * TB + tb) * 4 + r][lane];
    }
    __syncthreads();
  }
  if (wave < 4) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) s_acc[wave][(rt * TB + tb) * 4 + r][lane] = acc[rt][tb][r];
  }
  __syncthreads();
  if constexpr (kRopeTile) {
    if (a.rope) {
      // RoPE pairs (d, d + 64) of the tile's head: the quads of row tiles rt
      // and rt + RT / 2 (rt < RT / 2); rotation as in the separate RoPE kernel
      constexpr int kPairs = (RT / 2) * TB * 64;
#pragma unroll
      for (int q0 = 0; q0 < kPairs; q0 += 64 * NW) {
        const int q = q0 + tid;
        if (q >= kPairs) break;
        const int ql = q & 63, blk = q >> 6;    // blk = rt * TB + tb, rt < 4
        const int rt = blk / TB, tb = blk % TB;
        const int blk2 = blk + (RT / 2) * TB;
        float v1[4], v2[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v1[r] = ((s_acc[0][blk * 4 + r][ql] + s_acc[1][blk * 4 + r][ql]) + s_acc[2][blk * 4 + r][ql]) +
                  s_acc[3][blk * 4 + r][ql];
          v2[r] = ((s_acc[0][blk2 * 4 + r][ql] + s_acc[1][blk2 * 4 + r][ql]) + s_acc[2][blk2 * 4 + r][ql]) +
                  s_acc[3][blk2 * 4 + r][ql];
        }
        const int m = m0 + tb * 16 + (ql & 15);
        if (m >= a.M) continue;
        const int head = row16(0) / 8;
        const int d0 = (row16(rt) % 8) * 16 + (ql >> 4) * 4;  // < 64
        const int b = m / a.Lq, i = m % a.Lq;
        const int k = q0 / (64 * NW);                  // the prefetched values
        const int pos = (kEpiPf ? pf_p[k] : a.prefix_len[b]) + i;
        if (head >= a.Hq && pos >= a.Tmax) continue;   // past the cache: not written
        float o1[4], o2[4];
        bf16_t* dst;
        if (head < a.Hq + a.Hkv) {
          const float sc = head < a.Hq ? a.q_scale : 1.f;
          float4 cs4[2];
          if constexpr (kEpiPf) {
            cs4[0] = pf_cs[k][0];
            cs4[1] = pf_cs[k][1];
          } else {
            const float4* t = reinterpret_cast<const float4*>(a.rope_tab + static_cast<int64_t>(m) * 64 + d0);
            cs4[0] = t[0];
            cs4[1] = t[1];
          }
          const float cs[8] = {cs4[0].x, cs4[0].y, cs4[0].z, cs4[0].w, cs4[1].x, cs4[1].y, cs4[1].z, cs4[1].w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float c = cs[2 * r], sn = cs[2 * r + 1];
            o1[r] = (v1[r] * c - v2[r] * sn) * sc;
            o2[r] = (v2[r] * c + v1[r] * sn) * sc;
          }
          if (head < a.Hq) {
            const int G = a.Hq / a.Hkv;
            const int64_t row = static_cast<int64_t>(i) * G + head % G;
            dst = a.q_out + ((static_cast<int64_t>(b) * a.Hkv + head / G) * a.Lq * G + row) * 128;
          } else {
            dst = a.k_cache + ((static_cast<int64_t>(b) * a.Hkv + (head - a.Hq)) * a.Tmax + pos) * 128;
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) { o1[r] = v1[r]; o2[r] = v2[r]; }
          dst = a.v_cache +
                ((static_cast<int64_t>(b) * a.Hkv + (head - a.Hq - a.Hkv)) * a.Tmax + pos) * 128;
        }
        *reinterpret_cast<uint2*>(dst + d0) = make_uint2(pack_bf16x2(o1[0], o1[1]), pack_bf16x2(o1[2], o1[3]));
        *reinterpret_cast<uint2*>(dst + d0 + 64) =
            make_uint2(pack_bf16x2(o2[0], o2[1]), pack_bf16x2(o2[2], o2[3]));
      }
      return;
    }
  }
  constexpr int kQuads = RT * TB * 64;          // (row tile, token block, lane) quads
#pragma unroll
  for (int q0 = 0; q0 < kQuads; q0 += 64 * NW) {
    const int q = q0 + tid;
    if (q >= kQuads) break;
    const int ql = q & 63, blk = q >> 6;        // blk = rt * TB + tb
    const int rt = blk / TB, tb = blk % TB;
    const int n = n0 + rt * 16 + (ql >> 4) * 4;
    const int m = m0 + tb * 16 + (ql & 15);
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      v[r] = ((s_acc[0][blk * 4 + r][ql] + s_acc[1][blk * 4 + r][ql]) + s_acc[2][blk * 4 + r][ql]) +
             s_acc[3][blk * 4 + r][ql];
    }
    if (m >= a.M) continue;
    if (a.out_dtype == DG_F32) {
      float* o = static_cast<float*>(a.out) + static_cast<int64_t>(m) * a.N + n;
      if (a.accumulate) {
        const float4 c = kEpiPf ? pf_c[q0 / (64 * NW)] : *reinterpret_cast<const float4*>(o);
        *reinterpret_cast<float4*>(o) = make_float4(c.x + v[0], c.y + v[1], c.z + v[2], c.w + v[3]);
      } else {
        *reinterpret_cast<float4*>(o) = make_float4(v[0], v[1], v[2], v[3]);
      }
    } else {
      bf16_t* o = static_cast<bf16_t*>(a.out) + static_cast<int64_t>(m) * a.N + n;
      uint2 pk;
      pk.x = pack_bf16x2(v[0], v[1]);
      pk.y = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2*>(o) = pk;
    }
  }
}

}  // namespace dg

namespace dg {

// Dense GEMM for a thousand tokens and more (prefill chunks, the canvas of
// several rows) over tiled weights and tiled activations:
// out[m, n] = sum_k X[m, k] W[n, k].  A workgroup of four waves owns 128
// weight rows x 128 tokens over the whole K, so each operand byte it moves
// serves 128 outputs (the split-K tiles above move 720 KB per 64 x 64 tile at
// 256 tokens; here a 2048-token QKV projection moves half the bytes per
// output and runs in 52 against 111 us).  Per 64-k stage the 8 weight tiles'
// and the 8 token blocks' 2 KB chunks are copied into LDS unchanged by
// direct-to-LDS 16-byte loads (both tiled layouts already hold the MFMA
// operand lane order); NS stages are in flight.  Wave (wr, wt) owns rows
// 64 wr .. +64 and tokens 64 wt .. +64 (16 accumulator blocks).
// Epilogues: bf16 or f32 stores, f32 accumulate, or (a.rope) the QKV form:
// a 128-row tile is one head, wave wr = 1 hands its rows (d + 64) to wave
// wr = 0 through LDS, which rotates the pairs (angles from a.rope_tab) and
// writes q / k / v.
constexpr int kDl128Stage = 16384;               // elements per stage (32 KB)

template <int NS>
__global__ __launch_bounds__(256, 2) void gemm_dl128_kernel(GemmArgs a) {
  static_assert(NS >= 2 && NS * kDl128Stage * 2 >= 32 * 1024, "the RoPE hand-over fits a stage");
  extern __shared__ __attribute__((aligned(16))) bf16_t dl128_smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int logical = xcd_logical_tile(blockIdx.x, gridDim.x);
  if (logical >= a.n_tiles_total || step_gate_closed(a.gate, a.gate_n)) return;
  const int tx = logical / a.n_tiles_y, ty = logical % a.n_tiles_y;
  const int n0 = tx * 128, m0 = ty * 128;
  const int nch = a.K / 64;
  const int wr = wave & 1, wt = wave >> 1;
  const bf16_t* W = static_cast<const bf16_t*>(a.W);
  const int mblocks = (a.M + 15) / 16;
  // this wave's eight 1 KB blocks of every stage: block b = 8 wave + i is
  // half b % 2 of weight tile b / 2 (b < 16) or of token block (b - 16) / 2;
  // token blocks past the last one are clamped to it (their rows are masked
  // in the epilogue)
  const bf16_t* src[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int b = wave * 8 + i;
    if (b < 16) {
      src[i] = W + static_cast<int64_t>(n0 / 16 + (b >> 1)) * nch * 1024 + (b & 1) * 512 + lane * 8;
    } else {
      const int blk = min(m0 / 16 + ((b - 16) >> 1), mblocks - 1);
      src[i] = a.X + static_cast<int64_t>(blk) * nch * 1024 + (b & 1) * 512 + lane * 8;
    }
  }
  auto issue = [&](int c) {
    bf16_t* dst = dl128_smem + (c % NS) * kDl128Stage + wave * 8 * 512;
#pragma unroll
    for (int i = 0; i < 8; ++i) __builtin_amdgcn_global_load_lds(src[i] + c * 1024, dst + i * 512, 16, 0, 0);
  };
  f32x4_v acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < NS - 1; ++c)
    if (c < nch) issue(c);
  for (int c = 0; c < nch; ++c) {
    // stage c's copies have landed when at most the later stages' (8 each)
    // are outstanding; then every wave's have (barrier), and every wave is
    // done with stage c - 1, whose buffer the next issue refills.  A bare
    // barrier: the fence of __syncthreads would wait for every copy in flight
    if (c + NS - 2 < nch) __builtin_amdgcn_s_waitcnt(waitcnt_vm((NS - 2) * 8));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_barrier();
    if (c + NS - 1 < nch) issue(c + NS - 1);
    const bf16_t* st = dl128_smem + (c % NS) * kDl128Stage;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x8_v wa[4], xb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wa[i] = *reinterpret_cast<const bf16x8_v*>(st + ((wr * 4 + i) * 2 + h) * 512 + lane * 8);
        xb[i] = *reinterpret_cast<const bf16x8_v*>(st + (16 + (wt * 4 + i) * 2 + h) * 512 + lane * 8);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[i], xb[j], acc[i][j], 0, 0, 0);
    }
  }

  // lane: rows 4 g4 + r of row block i, token l16 of token block j
  if (a.rope) {
    // the rotating waves' cache lengths and (cos, sin), read before the
    // hand-over so that they arrive while it runs
    int pf_p[4];
    float4 pf_cs[4][4][2];
    if (wr == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = min(m0 + (wt * 4 + j) * 16 + l16, a.M - 1);
        pf_p[j] = a.prefix_len[m / a.Lq];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4* t = reinterpret_cast<const float4*>(a.rope_tab + static_cast<int64_t>(m) * 64 + i * 16 + g4 * 4);
          pf_cs[j][i][0] = t[0];
          pf_cs[j][i][1] = t[1];
        }
      }
    }
    // hand rows 64 .. 127 (the d + 64 halves of the head's pairs) to wave wr = 0
    __syncthreads();                             // every wave is done with the stages
    f32x4_v* s_x = reinterpret_cast<f32x4_v*>(dl128_smem);
    if (wr == 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) s_x[((wt * 4 + i) * 4 + j) * 64 + lane] = acc[i][j];
    }
    __syncthreads();
    if (wr == 1) return;
    const int head = tx;
    const int G = a.Hq / a.Hkv;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + (wt * 4 + j) * 16 + l16;
      if (m >= a.M) continue;
      const int b = m / a.Lq, i_tok = m % a.Lq;
      const int pos = pf_p[j] + i_tok;
      if (head >= a.Hq && pos >= a.Tmax) continue;   // past the cache: not written
      bf16_t* dst;
      if (head < a.Hq) {
        const int64_t row = static_cast<int64_t>(i_tok) * G + head % G;
        dst = a.q_out + ((static_cast<int64_t>(b) * a.Hkv + head / G) * a.Lq * G + row) * 128;
      } else if (head < a.Hq + a.Hkv) {
        dst = a.k_cache + ((static_cast<int64_t>(b) * a.Hkv + (head - a.Hq)) * a.Tmax + pos) * 128;
      } else {
        dst = a.v_cache + ((static_cast<int64_t>(b) * a.Hkv + (head - a.Hq - a.Hkv)) * a.Tmax + pos) * 128;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4_v v1 = acc[i][j];
        const f32x4_v v2 = s_x[((wt * 4 + i) * 4 + j) * 64 + lane];
        const int d0 = i * 16 + g4 * 4;            // < 64
        float o1[4], o2[4];
        if (head < a.Hq + a.Hkv) {
          const float sc = head < a.Hq ? a.q_scale : 1.f;
          const float4 c01 = pf_cs[j][i][0], c23 = pf_cs[j][i][1];   // (cos, sin) of d0 .. d0 + 3
          const float cs[8] = {c01.x, c01.y, c01.z, c01.w, c23.x, c23.y, c23.z, c23.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float c = cs[2 * r], sn = cs[2 * r + 1];
            o1[r] = (v1[r] * c - v2[r] * sn) * sc;
            o2[r] = (v2[r] * c + v1[r] * sn) * sc;
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) { o1[r] = v1[r]; o2[r] = v2[r]; }
        }
        *reinterpret_cast<uint2*>(dst + d0) = make_uint2(pack_bf16x2(o1[0], o1[1]), pack_bf16x2(o1[2], o1[3]));
        *reinterpret_cast<uint2*>(dst + d0 + 64) =
            make_uint2(pack_bf16x2(o2[0], o2[1]), pack_bf16x2(o2[2], o2[3]));
      }
    }
    return;
  }
  // the accumulate form's residual, every piece read before the first store
  // (each read would otherwise wait behind the stores before it)
  float4 pf_c[4][4];
  if (a.accumulate && a.out_dtype == DG_F32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = min(m0 + (wt * 4 + j) * 16 + l16, a.M - 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = n0 + (wr * 4 + i) * 16 + g4 * 4;
        pf_c[j][i] = *reinterpret_cast<const float4*>(static_cast<const float*>(a.out) + static_cast<int64_t>(m) * a.N + n);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + (wt * 4 + j) * 16 + l16;
    if (m >= a.M) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = n0 + (wr * 4 + i) * 16 + g4 * 4;
      const f32x4_v v = acc[i][j];
      if (a.out_dtype == DG_F32) {
        float* o = static_cast<float*>(a.out) + static_cast<int64_t>(m) * a.N + n;
        if (a.accumulate) {
          const float4 c4 = pf_c[j][i];
          *reinterpret_cast<float4*>(o) = make_float4(c4.x + v[0], c4.y + v[1], c4.z + v[2], c4.w + v[3]);
        } else {
          *reinterpret_cast<float4*>(o) = make_float4(v[0], v[1], v[2], v[3]);
        }
      } else {
        bf16_t* o = static_cast<bf16_t*>(a.out) + static_cast<int64_t>(m) * a.N + n;
        *reinterpret_cast<uint2*>(o) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
    }
  }
}

}  // namespace dg
