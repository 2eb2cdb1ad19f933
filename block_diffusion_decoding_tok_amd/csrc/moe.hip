// Sparse MoE feed-forward: top-k router, expert-sorted grouped GEMMs, combine.
//
// What is computed: only the experts selected for a token run on it (test.we0
// article, "26B MoE 설계가 의미하는 것"); the router takes the top-k logits
// (ties to the lower expert id) and the gates are the softmax of the selected
// logits; each expert is a gated FFN (GELU(u Wg^T) * (u Wu^T)) Wd^T; the token
// output is the gate-weighted sum of its k slots in slot order.
//
// Kernels:
//   route_topk_kernel   16 lanes per token: k rounds of a group-wide
//                       (logit desc, id asc) max; gates in float.
//   route_sort_kernel   one 1024-thread workgroup: histogram, exclusive scan
//                       -> expert_offsets, stable scatter of the slot entries
//                       t * k + j by expert (ballot-based ranks, deterministic).
//   route_fused_kernel  both in one workgroup, up to 64 tokens.
//   gemm_stream_kernel  (gemm_mfma.h) gate/up + GELU*up -> h [T*k, I] bf16 in
//                       sorted order; down + gate -> y_slot [T*k, D] bf16.
//   combine_kernel      y[t] += sum_j y_slot[t*k + j] in slot order.
//   f32 path            plain SIMT kernels over the same tables (parity path).
#include <algorithm>

#include "common.h"
#include "gemm_mfma.h"
#include "kernels.h"

namespace dg {

// ------------------------------------------------------------------ router
// Top-k of one token by a 16-lane group: sub-lane sl holds experts sl,
// sl + 16, ... (E <= 256); each of the k rounds takes the group-wide
// (logit desc, id asc) maximum of the experts not yet taken (four DPP
// steps).  Lane j < k of the group writes slot j: its id and its gate, the
// softmax of the k selected logits (sum in slot order).  QN = 16-lane rows of
// experts held per lane: 8 for E <= 128, else 16.
template <int QN>
__device__ __forceinline__ void route_load_logits(const float* row, int E, int sl, float (&v)[QN]) {
#pragma unroll
  for (int q = 0; q < QN; ++q) v[q] = row[min(q * 16 + sl, E - 1)];
}

// Ranks the logits v (as loaded by route_load_logits) of token t; with
// ids_lds the slot ids are also written there.
template <int QN>
__device__ __forceinline__ void route_rank(float (&v)[QN], int t, int E, int k, int sl,
                                           int32_t* __restrict__ ids, float* __restrict__ gates,
                                           int* ids_lds = nullptr) {
#pragma unroll
  for (int q = 0; q < QN; ++q)
    if (q * 16 + sl >= E) v[q] = -INFINITY;
  uint32_t taken = 0;
  float my_val = 0.f, best0 = 0.f, z = 0.f;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    float best = -INFINITY;
    int bid = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < QN; ++q) {    // branch-free: compares and selects
      const int e = q * 16 + sl;
      const bool ok = (e < E) & !((taken >> q) & 1u);
      const bool better = ok & ((v[q] > best) | ((v[q] == best) & (e < bid)));
      best = better ? v[q] : best;
      bid = better ? e : bid;
    }
    row16_max_lowid(best, bid);
    if ((bid & 15) == sl) taken |= 1u << (bid >> 4);
    if (j == 0) best0 = best;
    z += expf(best - best0);
    if (sl == j) { my_val = best; my_id = bid; }
  }
  if (sl < k) {
    ids[static_cast<int64_t>(t) * k + sl] = my_id;
    gates[static_cast<int64_t>(t) * k + sl] = expf(my_val - best0) / z;
    if (ids_lds) ids_lds[t * k + sl] = my_id;
  }
}

template <int QN>
__device__ __forceinline__ void route_topk_group(const float* row, int t, int E, int k, int sl,
                                                 int32_t* __restrict__ ids,
                                                 float* __restrict__ gates) {
  // the token's E logits; all QN loads issued unconditionally (clamped),
  // masked afterwards
  float v[QN];
  route_load_logits<QN>(row, E, sl, v);
  route_rank<QN>(v, t, E, k, sl, ids, gates);
}

// Four tokens per one-wave workgroup (spread over many CUs: the rounds are
// latency-bound).
template <int QN>
__global__ __launch_bounds__(64) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                        int E, int k, int32_t* __restrict__ ids,
                                                        float* __restrict__ gates) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 4);
  if (t >= T) return;
  route_topk_group<QN>(logits + static_cast<int64_t>(t) * E, t, E, k, threadIdx.x & 15, ids,
                       gates);
}

// Stable counting sort of the n = T * k slot entries by expert, by one
// 1024-thread workgroup.  Wave w owns the contiguous range of entries
// [w R, (w + 1) R), R = ceil(n / 16): it first counts its entries per expert
// (LDS atomic adds: the counts do not depend on the order), then -- after
// the counts are turned into each (wave, expert)'s first output position
// (experts ascending, waves ascending within an expert) -- walks its range
// in chunks of 64 and places every entry at that position plus its rank
// among the same expert's entries of the chunk (ballot-based).  Waves own
// ascending ranges and walk them in order, so equal experts keep the entry
// order t * k + j: the result is unique (deterministic).  The ballot match
// is the costly part (it runs on one CU), so it runs in the placement pass
// only, over the BITS bits that hold an id below E.
struct SortSmem {
  int cnt[16][256];       // per wave: entries per expert, then the running position
};

// Lanes of this wave whose expert equals mine (empty for an inactive lane);
// e < 2^BITS.
template <int BITS>
__device__ __forceinline__ uint64_t same_expert_lanes(int e, bool active) {
  uint64_t same = __ballot(active);
#pragma unroll
  for (int bit = 0; bit < BITS; ++bit) {
    const uint64_t bal = __ballot(active && ((e >> bit) & 1));
    same &= ((e >> bit) & 1) ? bal : ~bal;
  }
  return active ? same : 0ull;
}

template <int BITS>
__device__ void sort_slots(const int* ids, int n, int E, int32_t* __restrict__ offsets,
                           int32_t* __restrict__ sorted_rows, SortSmem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int q = tid; q < 16 * 256; q += 1024) (&sm.cnt[0][0])[q] = 0;
  __syncthreads();
  const int R = (n + 15) / 16;
  const int r0 = wave * R, r1 = min(n, r0 + R);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // pass 1: per-wave counts
  // (ids are clamped to [0, E): an id out of range can only misplace entries,
  // never address memory outside the tables)
  for (int i = r0 + lane; i < r1; i += 64) atomicAdd(&sm.cnt[wave][min(max(ids[i], 0), E - 1)], 1);
  __syncthreads();
  // positions: thread e < E turns its column into exclusive prefixes over the
  // waves; wave 0 then scans the experts' totals (4 per lane)
  int total = 0;
  if (tid < E) {
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const int c = sm.cnt[w][tid];
      sm.cnt[w][tid] = total;
      total += c;
    }
  }
  __shared__ int s_total[256];
  if (tid < 256) s_total[tid] = tid < E ? total : 0;
  __syncthreads();
  __shared__ int s_off[256];
  if (wave == 0) {
    int c[4], sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      c[q] = s_total[lane * 4 + q];
      sum += c[q];
    }
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int tt = __shfl_up(incl, o);
      if (lane >= o) incl += tt;
    }
    int run = incl - sum;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      if (e < E) { s_off[e] = run; offsets[e] = run; }
      run += c[q];
    }
    if (lane == 63) offsets[E] = incl;
  }
  __syncthreads();
  // pass 2: place the entries; the chunk's leader of each expert then moves
  // the wave's running position past the chunk's entries of that expert
  // (one wave's LDS accesses complete in issue order)
  for (int c0 = r0; c0 < r1; c0 += 64) {
    const int i = c0 + lane;
    const bool act = i < r1;
    const int e = act ? min(max(ids[i], 0), E - 1) : 0;
    const uint64_t same = same_expert_lanes<BITS>(e, act);
    const int rank = __popcll(same & below);
    const int pos = act ? s_off[e] + sm.cnt[wave][e] + rank : 0;
    if (act && pos < n) sorted_rows[pos] = i;
    if (act && rank == 0) sm.cnt[wave][e] += __popcll(same);
  }
}

// Up to kSortStage entries the ids are first copied into LDS, every thread
// issuing all its loads at once: the two passes then read LDS instead of
// paying a global-load latency per 64-entry chunk (15.7 -> 4 us at 8192
// entries).
constexpr int kSortStage = 16384;
constexpr int kSortStagePerThread = kSortStage / 1024;

__global__ __launch_bounds__(1024) void route_sort_kernel(const int32_t* __restrict__ ids, int n,
                                                          int E, int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ sorted_rows) {
  __shared__ SortSmem sm;
  if (n <= kSortStage) {
    __shared__ int s_ids[kSortStage];
    const int tid = threadIdx.x;
    int v[kSortStagePerThread];
#pragma unroll
    for (int j = 0; j < kSortStagePerThread; ++j) v[j] = ids[min(tid + j * 1024, n - 1)];
#pragma unroll
    for (int j = 0; j < kSortStagePerThread; ++j)
      if (tid + j * 1024 < n) s_ids[tid + j * 1024] = v[j];
    __syncthreads();
    if (E <= 128)
      sort_slots<7>(s_ids, n, E, offsets, sorted_rows, sm);
    else
      sort_slots<8>(s_ids, n, E, offsets, sorted_rows, sm);
  } else {
    if (E <= 128)
      sort_slots<7>(ids, n, E, offsets, sorted_rows, sm);
    else
      sort_slots<8>(ids, n, E, offsets, sorted_rows, sm);
  }
}

// The top-k and the sort in one 1024-thread workgroup, for up to
// kRouteFusedMaxTokens tokens (AR decode, small batches): 64 groups of 16
// lanes take the tokens g, g + 64, ..., the slot ids go to LDS as well, and
// the counting sort reads them there.  One launch instead of two.  The top-k
// rounds are VALU work (about 500 wave instructions per token): one CU takes
// the 256 tokens of a canvas step in ~15 us against ~1 us spread over 64 CUs,
// so canvas-sized and larger token counts keep the two launches.
constexpr int kRouteFusedMaxTokens = 64;
constexpr int kRouteFusedMax = kRouteFusedMaxTokens * 16;   // slot entries (k <= 16)

template <int QN>
__global__ __launch_bounds__(1024) void route_fused_kernel(const float* __restrict__ logits, int T,
                                                           int E, int k, int32_t* __restrict__ ids,
                                                           float* __restrict__ gates,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ sorted_rows) {
  __shared__ SortSmem sm;
  __shared__ int s_ids[kRouteFusedMax];
  const int g = threadIdx.x >> 4, sl = threadIdx.x & 15;
  if (g < T) {
    float v[QN];
    route_load_logits<QN>(logits + static_cast<int64_t>(g) * E, E, sl, v);
    for (int t = g; t < T; t += 64) {
      float cur[QN];
#pragma unroll
      for (int q = 0; q < QN; ++q) cur[q] = v[q];
      if (t + 64 < T) route_load_logits<QN>(logits + static_cast<int64_t>(t + 64) * E, E, sl, v);
      route_rank<QN>(cur, t, E, k, sl, ids, gates, s_ids);
    }
  }
  __syncthreads();
  if (E <= 128)
    sort_slots<7>(s_ids, T * k, E, offsets, sorted_rows, sm);
  else
    sort_slots<8>(s_ids, T * k, E, offsets, sorted_rows, sm);
}

size_t moe_route_workspace_bytes(int, int, int) { return 0; }

dg_status launch_moe_route(const float* logits, int T, int E, int k, int32_t* topk_ids,
                           float* gates, int32_t* offsets, int32_t* sorted_rows, void*,
                           hipStream_t stream) {
  if (T <= kRouteFusedMaxTokens) {
    if (E <= 128)
      route_fused_kernel<8><<<1, 1024, 0, stream>>>(logits, T, E, k, topk_ids, gates, offsets,
                                                    sorted_rows);
    else
      route_fused_kernel<16><<<1, 1024, 0, stream>>>(logits, T, E, k, topk_ids, gates, offsets,
                                                     sorted_rows);
    DG_LAUNCH_CHECK();
    return DG_OK;
  }
  if (E <= 128)
    route_topk_kernel<8><<<(T + 3) / 4, 64, 0, stream>>>(logits, T, E, k, topk_ids, gates);
  else
    route_topk_kernel<16><<<(T + 3) / 4, 64, 0, stream>>>(logits, T, E, k, topk_ids, gates);
  DG_LAUNCH_CHECK();
  route_sort_kernel<<<1, 1024, 0, stream>>>(topk_ids, T * k, E, offsets, sorted_rows);
  DG_LAUNCH_CHECK();
  return DG_OK;
}

// ------------------------------------------------------------- combine
template <typename TS>
__global__ void combine_kernel(const TS* __restrict__ y_slot, int T, int D, int k,
                               float* __restrict__ y) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;   // 4-wide
  const int64_t n4 = static_cast<int64_t>(T) * D / 4;
  if (idx >= n4) return;
  const int64_t t = idx / (D / 4), d4 = idx % (D / 4);
  float4 acc = reinterpret_cast<float4*>(y)[idx];
  for (int j = 0; j < k; ++j) {
    const TS* src = y_slot + (t * k + j) * D + d4 * 4;
    acc.x += Elem<TS>::load(src, 0);
    acc.y += Elem<TS>::load(src, 1);
    acc.z += Elem<TS>::load(src, 2);
    acc.w += Elem<TS>::load(src, 3);
  }
  reinterpret_cast<float4*>(y)[idx] = acc;
}

// ------------------------------------------------------------- f32 path
__global__ void gateup_f32_kernel(const float* __restrict__ x, const float* __restrict__ wgu,
                                  const int32_t* __restrict__ offsets,
                                  const int32_t* __restrict__ sorted_rows, int n_slots, int E,
                                  int D, int I, int k, float* __restrict__ h) {
  const int p = blockIdx.x;               // sorted position
  if (p >= n_slots) return;
  int e = 0;
  while (e < E - 1 && offsets[e + 1] <= p) ++e;
  const int t = sorted_rows[p] / k;
  const float* xr = x + static_cast<int64_t>(t) * D;
  for (int n = threadIdx.x; n < I; n += blockDim.x) {
    const float* wg = wgu + (static_cast<int64_t>(e) * 2 * I + n) * D;
    const float* wu = wgu + (static_cast<int64_t>(e) * 2 * I + I + n) * D;
    float g = 0.f, u = 0.f;
    for (int d = 0; d < D; ++d) { g = fmaf(xr[d], wg[d], g); u = fmaf(xr[d], wu[d], u); }
    h[static_cast<int64_t>(p) * I + n] = gelu_erf(g) * u;
  }
}

__global__ void down_f32_kernel(const float* __restrict__ h, const float* __restrict__ wd,
                                const int32_t* __restrict__ offsets,
                                const int32_t* __restrict__ sorted_rows,
                                const float* __restrict__ gates, int n_slots, int E, int D, int I,
                                float* __restrict__ y_slot) {
  const int p = blockIdx.x;
  if (p >= n_slots) return;
  int e = 0;
  while (e < E - 1 && offsets[e + 1] <= p) ++e;
  const int s = sorted_rows[p];
  const float g = gates[s];
  const float* hr = h + static_cast<int64_t>(p) * I;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    const float* w = wd + (static_cast<int64_t>(e) * D + d) * I;
    float acc = 0.f;
    for (int i = 0; i < I; ++i) acc = fmaf(hr[i], w[i], acc);
    y_slot[static_cast<int64_t>(s) * D + d] = g * acc;
  }
}

// ------------------------------------------------------------- launchers
// LDS-staged 64-token tiles (a thousand tokens and more): stages of 64 k, few
// in flight, so that many waves per SIMD stay resident (measured at 1024
// tokens: gate/up 190 -> 156 us, down 131 -> 94 us for two stages at four
// waves per SIMD against 128 k x 3 stages at two).  fp8 and MXFP4 weights:
// one weight stage in flight at five workgroups (20 waves) per CU, 96 VGPRs
// (prefill +1.8%, the batch-4 step +0.3% against two stages at four); bf16
// weights keep two stages at four (at five they spill).
constexpr int kMoeTB = 4;      // 64 tokens per tile
constexpr int kMoeKS = 1;      // 64 k per LDS stage
template <int WF> constexpr int moe_stream_pf() { return WF == kWBf16 ? 2 : 1; }
template <int WF> constexpr int moe_stream_minwg() { return WF == kWBf16 ? 1 : 5; }

size_t moe_ffn_workspace_bytes(int T, int D, int I, int E, int k, int x_dtype) {
  const size_t slots = static_cast<size_t>(T) * k;
  const size_t esz = x_dtype == DG_F32 ? 4 : 2;
  return align_up(slots * I * esz, 256) + align_up(slots * D * esz, 256);
}

// one-wave kernels: register ring depth (chunks of 64 k) and weight tiles of
// 16 rows per item; token tiles of 16 tokens, or of 32 for gate/up when the
// experts average 20 to 40 tokens (fewer items re-streaming the same rows).
// fp8 over 16-token tiles: one chunk in flight at four waves per SIMD, for
// gate/up (116 VGPRs; the 30-layer step +1.6% over two chunks at three waves)
// and down (128 rows per item, 118 VGPRs; the step +2.1% over 256 rows with
// two chunks at two waves)
constexpr int kMoeNR = 2, kMoeWPE = 3, kDownNR = 1, kDownWPE = 4;
constexpr int kGateNR = 1, kGateWPE = 4;
constexpr int kGateRT = 8;
constexpr int kDownRT = 8, kDownRTBf16 = 8;
constexpr int kGateTB1Slots = 20;   // gate/up: 16-token tiles up to this many slots per expert
constexpr int kTinySlots = 64;      // up to this many slots in all: half-size items

// MXFP4 weights: a chunk of a tile is half the bytes of fp8 (ring depth,
// waves per SIMD and weight tiles per item are set on their own; one chunk in
// flight at four waves per SIMD: the MXFP4 step +0.9% over two at three)
constexpr int kMx4NR = 1, kMx4WPE = 4;
constexpr int kMx4GateRT = 8, kMx4DownRT = 8;

template <int WF, int MODE>
constexpr int item_tiles() {
  return WF == kWMx4 ? (MODE == kGateUp ? kMx4GateRT : kMx4DownRT)
                     : (MODE == kGateUp ? kGateRT : (WF == kWFp8 ? kDownRT : kDownRTBf16));
}

// a handful of tokens (AR decode): few items, so each wave keeps a deeper ring
// of fewer weight tiles in flight
constexpr int kTinyRT = 2, kTinyNR = 4;

template <int TB, int WF, int MODE, bool TILED, int RT = item_tiles<WF, MODE>(), int NRT = 0>
static void launch_wave(GemmArgs& g, int T, int k, int E, hipStream_t stream) {
  // grid: an upper bound of the tile count times the weight row groups (an
  // expert with tokens has at most one partial tile, and at most min(E, T k)
  // experts have tokens); the kernel deals the live items out itself
  const int rows_per_item = MODE == kGateUp ? 8 * RT : 16 * RT;
  g.n_tiles_x = (MODE == kGateUp ? g.N / 2 : g.N) / rows_per_item;
  g.n_tiles_y = std::min(E, T * k) + (T * k + 16 * TB - 1) / (16 * TB);
  g.n_tiles_total = g.n_tiles_x * g.n_tiles_y;
  const unsigned grid = static_cast<unsigned>((g.n_tiles_total + 7) / 8 * 8);
  // bf16 chunks are twice the registers of fp8: two waves per SIMD (three
  // would spill the ring)
  if constexpr (NRT > 0)
    gemm_wave_kernel<RT, TB, NRT, WF, MODE, TILED, 1><<<grid, 64, 0, stream>>>(g);
  else if constexpr (WF == kWMx4)
    gemm_wave_kernel<RT, TB, kMx4NR, WF, MODE, TILED, (TB == 1 ? kMx4WPE : 1)><<<grid, 64, 0, stream>>>(g);
  else if constexpr (WF == kWBf16)
    gemm_wave_kernel<RT, TB, kMoeNR, WF, MODE, TILED, (TB == 1 ? 2 : 1)><<<grid, 64, 0, stream>>>(g);
  else
    gemm_wave_kernel<RT, TB, (MODE == kDown ? kDownNR : TB == 1 ? kGateNR : kMoeNR), WF, MODE, TILED,
                     (TB == 1 ? (MODE == kDown ? kDownWPE : kGateWPE) : 1)><<<grid, 64, 0, stream>>>(g);
}

// A tile-packed stack of E > 1 experts [E, N, K] (bf16 / fp8) keeps the k
// chunk c of every expert's 16-row tiles together: items streaming the same
// k range of different experts read neighbouring addresses.
static void stack_strides(GemmArgs& g, int N, int K, int E) {
  g.w_group_stride = static_cast<int64_t>(N / 16) * 1024;
  g.w_tile_stride = 1024;
  g.w_chunk_stride = static_cast<int64_t>(E) * (N / 16) * 1024;
}

// Bytes of one expert's weights [N, K] in format WF.
template <int WF>
static int64_t expert_bytes(int N, int K) {
  const int64_t nk = static_cast<int64_t>(N) * K;
  return WF == kWMx4 ? nk / 2 + nk / 32 : (WF == kWFp8 ? nk : 2 * nk);
}

template <int WF, bool TILED>
static void launch_gate_up_mfma(const void* x, const void* wgu, const float* sgu,
                                const int32_t* offsets, const int32_t* sorted_rows, int T, int D,
                                int I, int E, int k, bf16_t* h, hipStream_t stream,
                                const StepGate& gate) {
  GemmArgs g{};
  g.gate = gate.n_done;
  g.gate_n = gate.n;
  g.W = wgu;
  g.w_group_stride = WF == kWBf16 ? static_cast<int64_t>(2) * I * D : expert_bytes<WF>(2 * I, D);
  if (TILED && WF != kWMx4 && E > 1) stack_strides(g, 2 * I, D, E);
  g.w_scale = WF == kWFp8 ? sgu : nullptr; g.s_group_stride = 2 * I;
  g.X = static_cast<const bf16_t*>(x);
  g.N = 2 * I; g.K = D; g.n_groups = E; g.topk = k;
  g.offsets = offsets; g.sorted_rows = sorted_rows;
  g.out = h;
  // few tokens per expert (the canvas of one or two rows): one-wave items
  // streaming registers; more: 64-token tiles staged through LDS (every
  // weight format)
  const int64_t slots = static_cast<int64_t>(T) * k;
  if (slots <= kTinySlots) {
    // a few tokens (AR decode): half-size items, twice as many waves
    launch_wave<1, WF, kGateUp, TILED, kTinyRT, kTinyNR>(g, T, k, E, stream);
  } else if (slots <= kGateTB1Slots * static_cast<int64_t>(E)) {
    launch_wave<1, WF, kGateUp, TILED>(g, T, k, E, stream);
  } else if (slots <= 40ll * E) {
    launch_wave<2, WF, kGateUp, TILED>(g, T, k, E, stream);
  } else {
    const int MT = 16 * kMoeTB;
    g.n_tiles_x = I / 64;
    g.n_tiles_y = E + static_cast<int>((slots + MT - 1) / MT);
    g.n_tiles_total = g.n_tiles_x * g.n_tiles_y;
    gemm_stream_kernel<2, kMoeTB, kMoeKS, moe_stream_pf<WF>(), WF, kGateUp, TILED, moe_stream_minwg<WF>()>
        <<<(g.n_tiles_total + 7) / 8 * 8, 256, 0, stream>>>(g);
  }
}

template <int WF, bool TILED>
static void launch_down_mfma(const bf16_t* h, const void* wd, const float* sd, const float* gates,
                             const int32_t* offsets, const int32_t* sorted_rows, int T, int D,
                             int I, int E, int k, bf16_t* y_slot, hipStream_t stream,
                             const StepGate& gate) {
  GemmArgs d{};
  d.gate = gate.n_done;
  d.gate_n = gate.n;
  d.W = wd;
  d.w_group_stride = WF == kWBf16 ? static_cast<int64_t>(D) * I : expert_bytes<WF>(D, I);
  if (TILED && WF != kWMx4 && E > 1) stack_strides(d, D, I, E);
  d.w_scale = WF == kWFp8 ? sd : nullptr; d.s_group_stride = D;
  d.X = h;
  d.N = D; d.K = I; d.n_groups = E; d.topk = k;
  d.offsets = offsets; d.sorted_rows = sorted_rows; d.gates = gates;
  d.out = y_slot;
  const int64_t slots = static_cast<int64_t>(T) * k;
  if (slots <= kTinySlots) {
    launch_wave<1, WF, kDown, TILED, kTinyRT, kTinyNR>(d, T, k, E, stream);
  } else if (slots <= 40ll * E) {
    launch_wave<1, WF, kDown, TILED>(d, T, k, E, stream);
  } else {
    const int MT = 16 * kMoeTB;
    d.n_tiles_x = D / 128;
    d.n_tiles_y = E + static_cast<int>((slots + MT - 1) / MT);
    d.n_tiles_total = d.n_tiles_x * d.n_tiles_y;
    gemm_stream_kernel<2, kMoeTB, kMoeKS, moe_stream_pf<WF>(), WF, kDown, TILED, moe_stream_minwg<WF>()>
        <<<(d.n_tiles_total + 7) / 8 * 8, 256, 0, stream>>>(d);
  }
}

dg_status launch_moe_gate_up(const void* x, int x_dtype, const void* w_gate_up, int w_dtype,
                             int w_layout, const float* s_gate_up, const int32_t* offsets,
                             const int32_t* sorted_rows, int T, int D, int I, int E, int k,
                             void* h, hipStream_t stream, const StepGate& gate) {
  if (x_dtype == DG_F32) {
    gateup_f32_kernel<<<T * k, 128, 0, stream>>>(static_cast<const float*>(x),
                                                 static_cast<const float*>(w_gate_up), offsets,
                                                 sorted_rows, T * k, E, D, I, k,
                                                 static_cast<float*>(h));
    DG_LAUNCH_CHECK();
    return DG_OK;
  }
  const bool tiled = w_layout == DG_LAYOUT_TILED;
  bf16_t* hb = static_cast<bf16_t*>(h);
  if (w_dtype == DG_MXFP4) {
    launch_gate_up_mfma<kWMx4, true>(x, w_gate_up, nullptr, offsets, sorted_rows, T, D, I, E, k, hb, stream, gate);
  } else if (w_dtype == DG_FP8_E4M3) {
    if (tiled) launch_gate_up_mfma<kWFp8, true>(x, w_gate_up, s_gate_up, offsets, sorted_rows, T, D, I, E, k, hb, stream, gate);
    else launch_gate_up_mfma<kWFp8, false>(x, w_gate_up, s_gate_up, offsets, sorted_rows, T, D, I, E, k, hb, stream, gate);
  } else {
    if (tiled) launch_gate_up_mfma<kWBf16, true>(x, w_gate_up, nullptr, offsets, sorted_rows, T, D, I, E, k, hb, stream, gate);
    else launch_gate_up_mfma<kWBf16, false>(x, w_gate_up, nullptr, offsets, sorted_rows, T, D, I, E, k, hb, stream, gate);
  }
  DG_LAUNCH_CHECK();
  return DG_OK;
}

dg_status launch_moe_down(const void* h, int h_dtype, const void* w_down, int w_dtype,
                          int w_layout, const float* s_down, const float* gates,
                          const int32_t* offsets, const int32_t* sorted_rows, int T, int D, int I,
                          int E, int k, void* y_slot, hipStream_t stream, const StepGate& gate) {
  if (h_dtype == DG_F32) {
    down_f32_kernel<<<T * k, 128, 0, stream>>>(static_cast<const float*>(h),
                                               static_cast<const float*>(w_down), offsets,
                                               sorted_rows, gates, T * k, E, D, I,
                                               static_cast<float*>(y_slot));
    DG_LAUNCH_CHECK();
    return DG_OK;
  }
  const bool tiled = w_layout == DG_LAYOUT_TILED;
  const bf16_t* hb = static_cast<const bf16_t*>(h);
  bf16_t* yb = static_cast<bf16_t*>(y_slot);
  if (w_dtype == DG_MXFP4) {
    launch_down_mfma<kWMx4, true>(hb, w_down, nullptr, gates, offsets, sorted_rows, T, D, I, E, k, yb, stream, gate);
  } else if (w_dtype == DG_FP8_E4M3) {
    if (tiled) launch_down_mfma<kWFp8, true>(hb, w_down, s_down, gates, offsets, sorted_rows, T, D, I, E, k, yb, stream, gate);
    else launch_down_mfma<kWFp8, false>(hb, w_down, s_down, gates, offsets, sorted_rows, T, D, I, E, k, yb, stream, gate);
  } else {
    if (tiled) launch_down_mfma<kWBf16, true>(hb, w_down, nullptr, gates, offsets, sorted_rows, T, D, I, E, k, yb, stream, gate);
    else launch_down_mfma<kWBf16, false>(hb, w_down, nullptr, gates, offsets, sorted_rows, T, D, I, E, k, yb, stream, gate);
  }
  DG_LAUNCH_CHECK();
  return DG_OK;
}

dg_status launch_moe_combine(const void* y_slot, int dtype, int T, int D, int k, float* y,
                             hipStream_t stream) {
  const int64_t n4 = static_cast<int64_t>(T) * D / 4;
  const unsigned cblocks = static_cast<unsigned>((n4 + 255) / 256);
  if (dtype == DG_F32)
    combine_kernel<float><<<cblocks, 256, 0, stream>>>(static_cast<const float*>(y_slot), T, D, k, y);
  else
    combine_kernel<bf16_t><<<cblocks, 256, 0, stream>>>(static_cast<const bf16_t*>(y_slot), T, D, k, y);
  DG_LAUNCH_CHECK();
  return DG_OK;
}

void moe_ffn_workspace_split(void* ws, int T, int I, int k, int x_dtype, void** h,
                             void** y_slot) {
  const size_t slots = static_cast<size_t>(T) * k;
  const size_t esz = x_dtype == DG_F32 ? 4 : 2;
  *h = ws;
  *y_slot = static_cast<char*>(ws) + align_up(slots * I * esz, 256);
}

dg_status launch_moe_ffn(const void* x, int x_dtype, const void* w_gate_up, const void* w_down,
                         int w_dtype, int w_layout, const float* s_gate_up, const float* s_down,
                         const int32_t* topk_ids, const float* gates, const int32_t* offsets,
                         const int32_t* sorted_rows, int T, int D, int I, int E, int k, float* y,
                         void* ws, hipStream_t stream) {
  void *h, *y_slot;
  moe_ffn_workspace_split(ws, T, I, k, x_dtype, &h, &y_slot);
  dg_status st = launch_moe_gate_up(x, x_dtype, w_gate_up, w_dtype, w_layout, s_gate_up, offsets,
                                    sorted_rows, T, D, I, E, k, h, stream);
  if (st != DG_OK) return st;
  st = launch_moe_down(h, x_dtype, w_down, w_dtype, w_layout, s_down, gates, offsets, sorted_rows,
                       T, D, I, E, k, y_slot, stream);
  if (st != DG_OK) return st;
  return launch_moe_combine(y_slot, x_dtype, T, D, k, y, stream);
}

}  // namespace dg
