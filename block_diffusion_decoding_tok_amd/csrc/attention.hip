// Canvas attention and KV commit.
//
// What is computed: every canvas position attends to every other canvas
// position and to the committed prefix held in the KV cache (GeekNews summary,
// "핵심 트레이드오프"; developer guide, "Block Autoregressive Diffusion"); the
// prompt is kept as cache and never sees the canvas (technical-report summary,
// "DiffusionGemma의 구성", block-diagonal mask).  Scores q.k / sqrt(dh),
// grouped-query heads, RoPE (rotate-half pairs, theta^(-2j/dh)) at absolute
// positions, rotated keys in the cache.
//
// Launch sequence:
//   1. rope_kernel (unless the QKV projection already did it in its
//      epilogue): per token (heads spread over the workgroup's threads),
//      rotates the block's q (into a packed workspace
//      [B, Hkv, Lq * G, dh], packed row r = token * G + (head % G); for the
//      bf16 path pre-multiplied by log2(e) / sqrt(dh), so that scores come
//      out of the MFMA in the log2 domain) and k (into cache slots
//      [P, P + Lq)), copies v into the cache.
//   2. bf16: attn_mfma_kernel, one workgroup per (row tile of 128, KV split,
//      b * Hkv), the row tiles of one (split, head) on the same XCD so
//      that they share its K/V tiles in one L2; eight waves: four row groups
//      of 32 packed rows x two halves of every 128-key tile (two waves per
//      SIMD), merged through LDS at the end; K tile [128 keys][dh] (rows in
//      MFMA order) and V tile [128 keys][dh] copied into LDS by direct-to-LDS
//      loads (double buffered), V^T fragments read by transposing LDS reads;
//      S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_16x16x32_bf16
//      so that the probabilities leave the S MFMA already in the B-operand
//      layout of the PV MFMA; the running maximum is raised lazily.
//      f32: attn_f32_kernel, one wave per (query, head) -- parity path.
//   3. attn_combine_kernel merges the KV splits (online-softmax merge).
#include "common.h"
#include "kernels.h"

namespace dg {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

// ---------------------------------------------------------------- RoPE / KV
template <typename T>
__global__ __launch_bounds__(256) void rope_kernel(
    const T* __restrict__ q, const T* __restrict__ k_new, const T* __restrict__ v_new,
    int64_t q_stride, int64_t kv_stride, T* __restrict__ q_out, T* __restrict__ k_cache,
    T* __restrict__ v_cache, const int32_t* __restrict__ prefix_len, int Lq, int Hq, int Hkv,
    int dh, int Tmax, float theta, float q_scale) {
  // one workgroup per token; thread (pair j, head lane hl) handles heads
  // hl, hl + lanes, ... of the query heads and then of the KV heads
  const int tok = blockIdx.x;          // b * Lq + i
  const int b = tok / Lq, i = tok % Lq;
  const int half = dh / 2;
  const int j = threadIdx.x % half;
  const int hl = threadIdx.x / half;
  const int lanes = blockDim.x / half;
  if (hl >= lanes) return;
  const int pos = prefix_len[b] + i;
  float c, s;
  rope_cos_sin(pos, j, dh, theta, &c, &s);
  const int G = Hq / Hkv;
  if (q_out) {
    const T* qt = q + static_cast<int64_t>(tok) * q_stride;
    for (int h = hl; h < Hq; h += lanes) {
      const float x1 = Elem<T>::load(qt, h * dh + j), x2 = Elem<T>::load(qt, h * dh + j + half);
      const int g = h / G;
      const int64_t r = static_cast<int64_t>(i) * G + (h % G);
      T* dst = q_out + ((static_cast<int64_t>(b) * Hkv + g) * Lq * G + r) * dh;
      Elem<T>::store(dst, j, (x1 * c - x2 * s) * q_scale);
      Elem<T>::store(dst, j + half, (x2 * c + x1 * s) * q_scale);
    }
  }
  const T* kt = k_new + static_cast<int64_t>(tok) * kv_stride;
  const T* vt = v_new + static_cast<int64_t>(tok) * kv_stride;
  if (pos >= Tmax) return;             // past the cache: nothing is written
  for (int g = hl; g < Hkv; g += lanes) {
    const float x1 = Elem<T>::load(kt, g * dh + j), x2 = Elem<T>::load(kt, g * dh + j + half);
    const int64_t o = ((static_cast<int64_t>(b) * Hkv + g) * Tmax + pos) * dh;
    Elem<T>::store(k_cache + o, j, x1 * c - x2 * s);
    Elem<T>::store(k_cache + o, j + half, x2 * c + x1 * s);
    v_cache[o + j] = vt[g * dh + j];
    v_cache[o + j + half] = vt[g * dh + j + half];
  }
}

static int rope_threads(int dh) {
  const int half = dh / 2;
  return (256 / half) * half;          // a whole number of head lanes
}

__global__ void advance_prefix_kernel(int32_t* prefix_len, int B, int L) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) prefix_len[b] += L;
}

// ------------------------------------------------------------ bf16 MFMA path
constexpr int kAttnRows = 128;        // packed rows per workgroup (4 row groups of 32)
constexpr int kAttnKeys = 128;        // keys per LDS tile (2 halves of 64)
constexpr int kDh = 128;
constexpr int kKStride = kDh;         // K tile row stride (elements): 256 B, 16-byte pieces XOR-swizzled
constexpr int kVStride = kDh;         // V tile row stride (elements): 256 B, 16-byte pieces XOR-swizzled
constexpr int kKTileElems = kAttnKeys * kKStride;
constexpr int kVTileElems = kAttnKeys * kVStride;
// A row's running maximum is raised only when a tile's maximum exceeds it by
// more than this (log2 units): probabilities then stay below 2^8, and the
// rescale of the output accumulators is skipped on most tiles.
constexpr float kLazyRescale = 8.f;
// The row sums of P come from two more MFMAs per tile against a block of
// ones (the sum of the bf16 P the PV product uses) instead of 32 vector adds
// per lane and two cross-lane sums (calls 2% faster at batch 1 and 4;
// starting the S accumulators at minus the exponent base, to save the 32
// subtractions too, measured no faster).
constexpr bool kAttnMfmaRowSum = true;

// Block-causal masks: token i of a block of Lq sees the cache and the block's
// tokens up to the end of its own group of mask_blk (1: causal).
__device__ __forceinline__ int attn_block_end(int tok, int mask_blk, int Lq) {
  return min(Lq, (tok / mask_blk + 1) * mask_blk);
}

// Key held by LDS row r (0..127) of a K tile.  The S^T MFMA's output row
// 16 b + 4 g + r' (b = 0..3 within a 64-key half, g = lane / 16) must hold
// key 8 g + 4 (b & 1) + r' of the half's 32-key chunk b / 2, so that each
// lane's eight probabilities of a chunk are eight consecutive keys -- the
// B-operand layout of the PV MFMA over V^T in natural key order.  Keys are
// stored in that MFMA row order: within 32 rows, row bits (4, 3, 2) hold key
// bits (2, 4, 3).
__device__ __forceinline__ int k_row_key(int r) {
  return (r & ~31) | (((r >> 3) & 1) << 4) | (((r >> 2) & 1) << 3) | (((r >> 4) & 1) << 2) | (r & 3);
}

struct AttnPartialML { float m, l; };

// Maximum of x over the four lanes l16 + 16 g (g = 0..3) that hold one row's
// scores: a swap across the two 32-lane halves, then across neighbouring
// 16-lane rows (VALU lane swaps; a shuffle would take two LDS round trips).
// The NaN-propagating maximum needs no operand canonicalization (the
// number-preferring one doubles the VALU count on scores fresh from the MFMA).
__device__ __forceinline__ float fmax2(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float max_over_g4(float x) {
  const unsigned u = __float_as_uint(x);
  const auto h = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float a = fmax2(__uint_as_float(h[0]), __uint_as_float(h[1]));
  const unsigned ua = __float_as_uint(a);
  const auto r = __builtin_amdgcn_permlane16_swap(ua, ua, false, false);
  return fmax2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// K: the tile's 128 rows of 256 B copied straight into LDS by direct-to-LDS
// 16-byte loads (no staging registers): LDS row r holds key k_row_key(r),
// its 16-byte piece p in slot p ^ (r & 15), so that the 16 rows one
// S-fragment read touches use 16 different slots (no bank conflicts without
// row padding).  A wave instruction fills 1 KB (4 rows: lane i writes row
// i / 16, slot i % 16); eight waves issue four each.  Keys past the last
// valid one are clamped to it.
__device__ __forceinline__ void attn_issue_k(bf16_t* sk, const bf16_t* kbase, int key0, int k_end,
                                             int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (wave * 4 + i) * 4 + (lane >> 4);
    const int piece = (lane & 15) ^ (row & 15);
    const int gk = min(key0 + k_row_key(row), k_end - 1);
    __builtin_amdgcn_global_load_lds(kbase + static_cast<int64_t>(gk) * kDh + piece * 8,
                                     sk + (wave * 4 + i) * 4 * kKStride, 16, 0, 0);
  }
}

// V: the tile's 128 key rows of 256 B in natural order, copied into LDS the
// same way, piece p of row r in slot p ^ v_swz(r).  The PV MFMA's A operand
// is V^T (lane (l16, g4): dh l16 of a 16-row block, 8 consecutive keys);
// two transposing LDS reads (ds_read_b64_tr_b16) give it: within a group of
// 16 lanes, lane m reads dh 4 (m & 3) .. + 3 of key m / 4 (of 4 keys), and
// lane l receives element l % 4 of lanes 4 j + l / 4 (j = 0..3), i.e. dh l of
// the 4 keys.  v_swz gives the 8 rows two groups read at once (keys 0..3 and
// 8..11 of a 16-key block) 8 different slot pairs.
__device__ __forceinline__ int v_swz(int r) { return ((r & 3) | (((r >> 3) & 1) << 2)) << 1; }
__device__ __forceinline__ void attn_issue_v(bf16_t* sv, const bf16_t* vbase, int key0, int k_end,
                                             int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (wave * 4 + i) * 4 + (lane >> 4);
    const int piece = (lane & 15) ^ v_swz(row);
    const int gk = min(key0 + row, k_end - 1);
    __builtin_amdgcn_global_load_lds(vbase + static_cast<int64_t>(gk) * kDh + piece * 8,
                                     sv + (wave * 4 + i) * 4 * kVStride, 16, 0, 0);
  }
}
// The V^T fragment of keys key0 .. key0 + 7 (key0 a multiple of 8, the
// lane's group's) and dh d0 + l16 (d0 a multiple of 16).
typedef short v4i16_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8_t attn_read_vt(const bf16_t* sv, int key0, int d0, int l16) {
  v4i16_t h[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int row = key0 + half * 4 + (l16 >> 2);
    const int col = d0 + 4 * (l16 & 3);
    const bf16_t* p = sv + row * kVStride + (((col >> 3) ^ v_swz(row)) << 3) + (col & 7);
    h[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)(p));
  }
  const v4i16_t lo = h[0], hi = h[1];
  typedef short v8i16_t __attribute__((ext_vector_type(8)));
  const v8i16_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}


__global__ __launch_bounds__(512) void attn_mfma_kernel(
    const bf16_t* __restrict__ qrot, const bf16_t* __restrict__ k_cache,
    const bf16_t* __restrict__ v_cache, const int32_t* __restrict__ prefix_len, int Lq, int G,
    int Hkv, int Tmax, int chunk, int ntile_rows, int nsplit, int BH, int mask_blk,
    float* __restrict__ o_part, AttnPartialML* __restrict__ ml_part, const int32_t* gate,
    int gate_n, const int32_t* __restrict__ row_done) {
  extern __shared__ __attribute__((aligned(16))) bf16_t smem[];
  // [K tile 0][K tile 1][V^T tile 0][V^T tile 1]
  auto s_k = [&](int buf) { return smem + buf * kKTileElems; };
  auto s_v = [&](int buf) { return smem + 2 * kKTileElems + buf * kVTileElems; };

  // logical index: row tile fastest, then split, then (b, kv head); workgroup
  // i runs on XCD i % 8, so consecutive logical indices are dealt to one XCD
  const int total = ntile_rows * nsplit * BH;
  const int logical = xcd_logical_tile(blockIdx.x, gridDim.x);
  if (logical >= total) return;
  const int tile = logical % ntile_rows;
  const int split = (logical / ntile_rows) % nsplit;
  const int bh = logical / (ntile_rows * nsplit);
  const int b = bh / Hkv;
  // the adaptive loop's gate: every row stopped, or this row stopped
  if (step_gate_closed(gate, gate_n) || (row_done && row_done[b])) return;
  const int rows_total = Lq * G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int rg = wave & 3, kh = wave >> 2;          // row group, key half
  const int P = prefix_len[b];
  const int n_keys = min(P + Lq, Tmax);             // never read past the cache
  const int row0 = tile * kAttnRows + rg * 32;      // this wave's first packed row

  // key range of this split: the row's keys [0, P + Lq) dealt out evenly in
  // whole tiles (P is read on the device, so a captured graph replayed at a
  // larger prefix still balances its splits; chunk * nsplit covers Tmax);
  // block-causal (mask_blk > 0): trimmed to the last row of the tile
  const int even = ((n_keys + nsplit - 1) / nsplit + kAttnKeys - 1) / kAttnKeys * kAttnKeys;
  const int split_keys = min(chunk, even);
  const int k_begin = split * split_keys;
  int k_end = min(n_keys, k_begin + split_keys);
  if (mask_blk) {
    const int last_row = min(rows_total - 1, tile * kAttnRows + kAttnRows - 1);
    k_end = min(k_end, P + attn_block_end(last_row / G, mask_blk, Lq));
  }
  const int ntiles = k_end > k_begin ? (k_end - k_begin + kAttnKeys - 1) / kAttnKeys : 0;

  // Q fragments (B operand of S^T = K Q^T): row l16 of each 16-row block,
  // dh 32c + 8 g4 .. +7; q is pre-scaled into the log2 domain
  bf16x8_t qf[2][4];
  const bf16_t* qbase = qrot + static_cast<int64_t>(bh) * rows_total * kDh;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int r = row0 + qb * 16 + l16;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (r < rows_total)
        qf[qb][c] = *reinterpret_cast<const bf16x8_t*>(qbase + static_cast<int64_t>(r) * kDh + c * 32 + g4 * 8);
      else
        qf[qb][c] = bf16x8_t{};
    }
  }
  int tok_of[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) tok_of[qb] = (row0 + qb * 16 + l16) / G;
  const int wave_tok = row0 / G;   // smallest token of the wave's rows

  f32x4_t acc_o[2][8];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int d = 0; d < 8; ++d) acc_o[qb][d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY};   // exponent base in use (per row)
  float l_run[2] = {0.f, 0.f};
  f32x4_t acc_l[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
  bf16x8_t ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = static_cast<__bf16>(1.0f);

  const bf16_t* kbase = k_cache + static_cast<int64_t>(bh) * Tmax * kDh;
  const bf16_t* vbase = v_cache + static_cast<int64_t>(bh) * Tmax * kDh;

  // K/V tiles in LDS double buffers, both filled by direct copies (no
  // staging registers).  Iteration t waits for its copies of tile t, then
  // (after the barrier) starts those of tile t + 1 into the other buffers,
  // which held tile t - 1, read before the barrier.
  if (ntiles > 0) {
    attn_issue_k(s_k(0), kbase, k_begin, k_end, wave, lane);
    attn_issue_v(s_v(0), vbase, k_begin, k_end, wave, lane);
  }
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    // this wave's copies of tile t have landed; after the barrier every wave's
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    if (t + 1 < ntiles) {
      attn_issue_k(s_k(buf ^ 1), kbase, k_begin + (t + 1) * kAttnKeys, k_end, wave, lane);
      attn_issue_v(s_v(buf ^ 1), vbase, k_begin + (t + 1) * kAttnKeys, k_end, wave, lane);
    }
    const int hkey0 = k_begin + t * kAttnKeys + kh * 64;   // first key of this wave's half
    const bf16_t* sk = s_k(buf) + kh * 64 * kKStride;
    const bf16_t* sv = s_v(buf);

    // S^T blocks [kb][qb]: MFMA row 4 g4 + r of block kb is key
    // 32 (kb / 2) + 8 g4 + 4 (kb & 1) + r of the half; column = row l16
    f32x4_t s_acc[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) s_acc[kb][qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(
            &sk[(kb * 16 + l16) * kKStride + ((c * 4 + g4) ^ l16) * 8]);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          s_acc[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[qb][c], s_acc[kb][qb], 0, 0, 0);
      }
    }
    // keys at or past a row's limit only occur in the split's last tile, or
    // past the wave's first token's block under a block-causal mask
    const int wave_lim = mask_blk ? min(k_end, P + attn_block_end(wave_tok, mask_blk, Lq)) : k_end;
    const bool edge = hkey0 + 64 > wave_lim;   // wave-uniform
    bf16x8_t pf[2][2];   // [qb][32-key chunk]
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      if (edge) {
        const int key_lim = mask_blk ? min(k_end, P + attn_block_end(tok_of[qb], mask_blk, Lq)) : k_end;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = hkey0 + (kb >> 1) * 32 + g4 * 8 + (kb & 1) * 4 + r;
            if (key >= key_lim) s_acc[kb][qb][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        mx = fmax2(fmax2(mx, s_acc[kb][qb][0]), s_acc[kb][qb][1]);
        mx = fmax2(fmax2(mx, s_acc[kb][qb][2]), s_acc[kb][qb][3]);
      }
      mx = max_over_g4(mx);
      // raise the base only past the lazy margin (wave-uniform decision)
      if (__any(mx > m_run[qb] + kLazyRescale)) {
        const float m_new = fmaxf(m_run[qb], mx);
        const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run[qb] - m_new);
        m_run[qb] = m_new;
        l_run[qb] *= alpha;
        acc_l[qb] *= alpha;
#pragma unroll
        for (int d = 0; d < 8; ++d) acc_o[qb][d] *= alpha;
      }
      const float base = (m_run[qb] == -INFINITY) ? 0.f : m_run[qb];
      float rs = 0.f;
      uint32_t pk[2][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[r] = __builtin_amdgcn_exp2f(s_acc[kb][qb][r] - base);
          if (!kAttnMfmaRowSum) rs += p[r];
        }
        pk[kb >> 1][(kb & 1) * 2 + 0] = pack_bf16x2(p[0], p[1]);
        pk[kb >> 1][(kb & 1) * 2 + 1] = pack_bf16x2(p[2], p[3]);
      }
      if (!kAttnMfmaRowSum) l_run[qb] += rs;
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
        uint4 u = make_uint4(pk[ch][0], pk[ch][1], pk[ch][2], pk[ch][3]);
        pf[qb][ch] = *reinterpret_cast<bf16x8_t*>(&u);
      }
    }
    // O^T[d] += V^T[d block][keys] P^T
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const bf16x8_t va = attn_read_vt(sv, kh * 64 + ch * 32 + g4 * 8, d * 16, l16);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          acc_o[qb][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pf[qb][ch], acc_o[qb][d], 0, 0, 0);
      }
      // row sums of P: every output row of ones . P^T is the column sum
      if (kAttnMfmaRowSum) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          acc_l[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[qb][ch], acc_l[qb], 0, 0, 0);
      }
    }
  }

  // ---- merge the two key halves of each row group through LDS, then write
  // the split's partial: O unnormalized [rows][dh] f32, (m, l) per row
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    if (kAttnMfmaRowSum) {
      l_run[qb] = acc_l[qb][0];            // the whole half's sum for row l16
    } else {
      l_run[qb] += __shfl_xor(l_run[qb], 16);
      l_run[qb] += __shfl_xor(l_run[qb], 32);
    }
  }
  __syncthreads();                       // every wave is done with the tiles
  // rows padded by 4 floats: the 16 rows a 16-lane group touches start on
  // different banks
  constexpr int kOStride = kDh + 4;
  float* s_o = reinterpret_cast<float*>(smem) + rg * (32 * kOStride + 64);
  float* s_ml = s_o + 32 * kOStride;
  if (kh == 1) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int d = 0; d < 8; ++d)
        *reinterpret_cast<f32x4_t*>(&s_o[(qb * 16 + l16) * kOStride + d * 16 + g4 * 4]) = acc_o[qb][d];
      if (g4 == 0) {
        s_ml[(qb * 16 + l16) * 2 + 0] = m_run[qb];
        s_ml[(qb * 16 + l16) * 2 + 1] = l_run[qb];
      }
    }
  }
  __syncthreads();
  if (kh == 1) return;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float m1 = s_ml[(qb * 16 + l16) * 2 + 0], l1 = s_ml[(qb * 16 + l16) * 2 + 1];
    const float M = fmaxf(m_run[qb], m1);
    const float base = (M == -INFINITY) ? 0.f : M;
    const float f0 = __builtin_amdgcn_exp2f(m_run[qb] - base), f1 = __builtin_amdgcn_exp2f(m1 - base);
    const float l = l_run[qb] * f0 + l1 * f1;
    const int r = row0 + qb * 16 + l16;
    if (r >= rows_total) continue;
    const int64_t prow = (static_cast<int64_t>(split) * BH + bh) * rows_total + r;
    float* dst = o_part + prow * kDh;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const f32x4_t o1 = *reinterpret_cast<const f32x4_t*>(&s_o[(qb * 16 + l16) * kOStride + d * 16 + g4 * 4]);
      *reinterpret_cast<float4*>(dst + d * 16 + g4 * 4) =
          make_float4(acc_o[qb][d][0] * f0 + o1[0] * f1, acc_o[qb][d][1] * f0 + o1[1] * f1,
                      acc_o[qb][d][2] * f0 + o1[2] * f1, acc_o[qb][d][3] * f0 + o1[3] * f1);
    }
    if (g4 == 0) ml_part[prow] = AttnPartialML{M, l};
  }
}

constexpr size_t kAttnSmemBytes = (2 * kKTileElems + 2 * kVTileElems) * sizeof(bf16_t);
static_assert(4 * (32 * (kDh + 4) + 64) * sizeof(float) <= kAttnSmemBytes, "merge scratch fits");

// ------------------------------------------------ few query rows (AR decode)
// Up to kDecRows packed rows per KV head (one token: the G heads of a group):
// the 128-row tiles above would be almost all padding, and their key tiles
// pass through LDS one after another.  Here a 512-thread workgroup owns an
// even share (a multiple of 64 keys) of one (b, kv head)'s keys; per chunk
// of kDecKeys each of its eight waves takes 64 keys and issues all of their
// K and V loads at once (pinned ahead of the arithmetic):
//   S^T = K Q^T on v_mfma_f32_16x16x32_bf16, the K rows straight from memory
//   as the A operand (lane (l16, g4): key l16 of a 16-key block, dh
//   32 c + 8 g4 .. + 7), q padded to 16 rows as B; lane (l16, g4) then holds
//   the scores of keys 16 kb + 4 g4 + r of row l16;
//   online softmax per row (maximum over the lane's 16 scores, then over the
//   four g4 lanes by lane swaps; the row's rescale factor broadcast from its
//   lane);
//   P V on the VALU: lane (l16, g4) accumulates dh 8 l16 .. + 7 of every row
//   over the keys 4 i + g4 (i = 0..15), the probabilities read from LDS;
// at the end the four g4 partial sums are added by lane swaps, the eight
// waves merge through LDS (online-softmax rescale) and the workgroup writes
// the split's partial in the layout attn_combine_kernel reads.
constexpr int kDecWaves = 8;
constexpr int kDecKeys = 64 * kDecWaves;   // keys per chunk (64 per wave)
constexpr int kDecRows = 4;
constexpr int kDecTargetWgs = 256;         // workgroups per launch (one per CU)

__device__ __forceinline__ float sum_over_g4(float x) {
  const unsigned u = __float_as_uint(x);
  const auto h = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float a = __uint_as_float(h[0]) + __uint_as_float(h[1]);
  const unsigned ua = __float_as_uint(a);
  const auto r = __builtin_amdgcn_permlane16_swap(ua, ua, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int RP>   // rows computed (>= the real row count R)
__global__ __launch_bounds__(64 * kDecWaves) void attn_decode_kernel(
    const bf16_t* __restrict__ qrot, const bf16_t* __restrict__ k_cache,
    const bf16_t* __restrict__ v_cache, const int32_t* __restrict__ prefix_len, int Lq, int G,
    int Hkv, int Tmax, int nsplit, int BH, int mask_blk, float* __restrict__ o_part,
    AttnPartialML* __restrict__ ml_part, const int32_t* gate, int gate_n,
    const int32_t* __restrict__ row_done) {
  static_assert(RP <= kDecRows, "rows");
  const int split = blockIdx.x % nsplit, bh = blockIdx.x / nsplit;
  if (bh >= BH) return;
  const int b = bh / Hkv;
  if (step_gate_closed(gate, gate_n) || (row_done && row_done[b])) return;
  const int R = Lq * G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int P = prefix_len[b];
  const int n_keys = min(P + Lq, Tmax);
  // keys any row of this head sees (block-causal: up to the last token's
  // block), dealt out evenly in whole chunks (P is read on the device, so a
  // captured graph replayed at a larger prefix still balances its splits)
  const int k_all = mask_blk ? min(n_keys, P + attn_block_end(Lq - 1, mask_blk, Lq)) : n_keys;
  const int share = ((k_all + nsplit - 1) / nsplit + 63) / 64 * 64;
  const int k_begin = split * share;
  const int k_end = min(k_all, k_begin + share);
  // this lane's row (rows past R repeat row R - 1's limit; they are not written)
  const int key_lim_row =
      mask_blk ? min(k_end, P + attn_block_end(min(l16, R - 1) / G, mask_blk, Lq)) : k_end;

  const bf16_t* kbase = k_cache + static_cast<int64_t>(bh) * Tmax * kDh;
  const bf16_t* vbase = v_cache + static_cast<int64_t>(bh) * Tmax * kDh;
  const bf16_t* qbase = qrot + static_cast<int64_t>(bh) * R * kDh;
  bf16x8_t qf[4];
  const int qrow = l16 < R ? l16 : 0;
#pragma unroll
  for (int c = 0; c < 4; ++c)
    qf[c] = *reinterpret_cast<const bf16x8_t*>(qbase + static_cast<int64_t>(qrow) * kDh + c * 32 + g4 * 8);
  if (l16 >= R) {
#pragma unroll
    for (int c = 0; c < 4; ++c) qf[c] = bf16x8_t{};
  }

  __shared__ float s_p[kDecWaves][64][RP];
  float m_run = -INFINITY;   // row l16's exponent base (log2 domain)
  float l_run = 0.f;         // this lane's share of row l16's sum
  float o[RP][8];
#pragma unroll
  for (int j = 0; j < RP; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[j][e] = 0.f;

  for (int kc = k_begin; kc < k_end; kc += kDecKeys) {
    const int k0 = kc + wave * 64;
    const int kw_end = min(k_end, k0 + 64);            // this wave's keys [k0, kw_end)
    const int k_last = max(min(kw_end, Tmax) - 1, 0);  // loads past it are clamped to it
    bf16x8_t kf[4][4];
    uint4 vr[16];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int key = min(k0 + kb * 16 + l16, k_last);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        kf[kb][c] = *reinterpret_cast<const bf16x8_t*>(kbase + static_cast<int64_t>(key) * kDh + c * 32 + g4 * 8);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = min(k0 + 4 * i + g4, k_last);
      vr[i] = *reinterpret_cast<const uint4*>(vbase + static_cast<int64_t>(key) * kDh + l16 * 8);
    }
    __builtin_amdgcn_sched_barrier(0);   // every load of the chunk issued first
    // scores (log2 domain: q carries log2(e) / sqrt(dh))
    f32x4_t sc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      sc[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        sc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kb][c], qf[c], sc[kb], 0, 0, 0);
    }
    const int key_lim = min(kw_end, key_lim_row);
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (k0 + kb * 16 + 4 * g4 + r >= key_lim) sc[kb][r] = -INFINITY;
        mx = fmax2(mx, sc[kb][r]);
      }
    mx = max_over_g4(mx);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    const float base = (m_new == -INFINITY) ? 0.f : m_new;
    l_run *= alpha;
#pragma unroll
    for (int j = 0; j < RP; ++j) {
      // row j's factor, from a lane that holds row j
      const float aj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), j));
#pragma unroll
      for (int e = 0; e < 8; ++e) o[j][e] *= aj;
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pv = __builtin_amdgcn_exp2f(sc[kb][r] - base);
        l_run += pv;
        if (l16 < RP) s_p[wave][kb * 16 + 4 * g4 + r][l16] = pv;
      }
    // (one wave's LDS writes complete before its later reads)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float vf[8];
      const uint32_t w[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        vf[2 * h] = __uint_as_float(w[h] << 16);
        vf[2 * h + 1] = __uint_as_float(w[h] & 0xffff0000u);
      }
#pragma unroll
      for (int j = 0; j < RP; ++j) {
        const float pj = s_p[wave][4 * i + g4][j];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[j][e] = __builtin_fmaf(pj, vf[e], o[j][e]);
      }
    }
  }
  l_run = sum_over_g4(l_run);
#pragma unroll
  for (int j = 0; j < RP; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[j][e] = sum_over_g4(o[j][e]);

  // merge the waves: row j's base and sum sit in lanes l16 = j
  __shared__ float s_m[kDecWaves][RP], s_l[kDecWaves][RP];
  __shared__ float s_o[kDecWaves][RP][kDh];
  if (g4 == 0) {
    if (l16 < RP) { s_m[wave][l16] = m_run; s_l[wave][l16] = l_run; }
#pragma unroll
    for (int j = 0; j < RP; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) s_o[wave][j][l16 * 8 + e] = o[j][e];
  }
  __syncthreads();
  for (int q = tid; q < R * kDh; q += 64 * kDecWaves) {
    const int j = q / kDh, d = q % kDh;
    float M = -INFINITY;
#pragma unroll
    for (int w2 = 0; w2 < kDecWaves; ++w2) M = fmaxf(M, s_m[w2][j]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < kDecWaves; ++w2) {
      const float f = s_m[w2][j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s_m[w2][j] - M);
      L += s_l[w2][j] * f;
      O += s_o[w2][j][d] * f;
    }
    const int64_t prow = (static_cast<int64_t>(split) * BH + bh) * R + j;
    o_part[prow * kDh + d] = O;
    if (d == 0) ml_part[prow] = AttnPartialML{M, L};
  }
}

// Merge the KV splits of every packed row and write out [B, Lq, Hq, dh]
// (row-major, or with tiled the tiled activation layout of [B Lq, Hq dh]):
// 32 threads per row (4 dh each, 16-byte loads), 8 rows per workgroup.
template <typename T>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ o_part,
                                                           const AttnPartialML* __restrict__ ml_part,
                                                           int nsplit, int BH, int rows_total,
                                                           int G, int Hkv, int Lq, int tiled,
                                                           T* __restrict__ out,
                                                           const int32_t* gate, int gate_n,
                                                           const int32_t* __restrict__ row_done) {
  const int gr = blockIdx.x * 8 + (threadIdx.x >> 5);      // global packed row index
  const int d4 = (threadIdx.x & 31) * 4;
  if (gr >= BH * rows_total || step_gate_closed(gate, gate_n)) return;
  const int bh = gr / rows_total, r = gr % rows_total;
  if (row_done && row_done[bh / Hkv]) return;
  // splits in batches of 8: a batch's (m, l) and O loads are issued together
  // (clamped indices, masked afterwards), then merged in split order with an
  // online rescale when a batch raises the running maximum (one pass)
  const int64_t rstride = static_cast<int64_t>(BH) * rows_total;
  const int64_t r0 = static_cast<int64_t>(bh) * rows_total + r;
  float M = -INFINITY;
  float L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < nsplit; s0 += 8) {
    AttnPartialML ml[8];
    float4 o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t prow = min(s0 + j, nsplit - 1) * rstride + r0;
      ml[j] = ml_part[prow];
      o[j] = *reinterpret_cast<const float4*>(o_part + prow * kDh + d4);
    }
    float mb = M;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s0 + j < nsplit && ml[j].l != 0.f) mb = fmaxf(mb, ml[j].m);
    if (mb > M) {                     // raise the base: rescale what is summed so far
      const float f = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M - mb);
      L *= f;
      acc.x *= f; acc.y *= f; acc.z *= f; acc.w *= f;
      M = mb;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (s0 + j >= nsplit || ml[j].l == 0.f) continue;
      const float f = __builtin_amdgcn_exp2f(ml[j].m - M);
      L += ml[j].l * f;
      acc.x += o[j].x * f;
      acc.y += o[j].y * f;
      acc.z += o[j].z * f;
      acc.w += o[j].w * f;
    }
  }
  const int b = bh / Hkv, g = bh % Hkv;
  const int tok = r / G, h = g * G + r % G;
  const int Hq = Hkv * G;
  const int64_t m = static_cast<int64_t>(b) * Lq + tok;
  T* dst = tiled ? out + xtile_offset(m, h * kDh + d4, Hq * kDh) : out + (m * Hq + h) * kDh + d4;
  Elem<T>::store(dst, 0, acc.x / L);
  Elem<T>::store(dst, 1, acc.y / L);
  Elem<T>::store(dst, 2, acc.z / L);
  Elem<T>::store(dst, 3, acc.w / L);
}

// The same merge for the decode kernel's few rows: one workgroup per packed
// row, its eight groups of 32 threads (4 dh each) take the splits g, g + 8,
// ... (loads issued together, online rescale), then the groups merge through
// LDS.  (With 32 threads per row the whole merge of one token ran on two
// workgroups, one split after another.)
template <typename T>
__global__ __launch_bounds__(256) void attn_combine_few_kernel(
    const float* __restrict__ o_part, const AttnPartialML* __restrict__ ml_part, int nsplit,
    int BH, int rows_total, int G, int Hkv, int Lq, int tiled, T* __restrict__ out,
    const int32_t* gate, int gate_n, const int32_t* __restrict__ row_done) {
  const int gr = blockIdx.x;                        // packed row (bh, r)
  if (gr >= BH * rows_total || step_gate_closed(gate, gate_n)) return;
  const int bh = gr / rows_total, r = gr % rows_total;
  if (row_done && row_done[bh / Hkv]) return;
  const int grp = threadIdx.x >> 5, d4 = (threadIdx.x & 31) * 4;
  const int64_t rstride = static_cast<int64_t>(BH) * rows_total;
  const int64_t r0 = static_cast<int64_t>(bh) * rows_total + r;
  float M = -INFINITY, L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = grp; s0 < nsplit; s0 += 32) {
    AttnPartialML ml[4];
    float4 o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t prow = min(s0 + 8 * j, nsplit - 1) * rstride + r0;
      ml[j] = ml_part[prow];
      o[j] = *reinterpret_cast<const float4*>(o_part + prow * kDh + d4);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (s0 + 8 * j >= nsplit || ml[j].l == 0.f) continue;
      const float mb = fmaxf(M, ml[j].m);
      const float f0 = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M - mb);
      const float f1 = __builtin_amdgcn_exp2f(ml[j].m - mb);
      L = L * f0 + ml[j].l * f1;
      acc.x = acc.x * f0 + o[j].x * f1;
      acc.y = acc.y * f0 + o[j].y * f1;
      acc.z = acc.z * f0 + o[j].z * f1;
      acc.w = acc.w * f0 + o[j].w * f1;
      M = mb;
    }
  }
  __shared__ float s_m[8], s_l[8];
  __shared__ float4 s_acc[8][32];
  if ((threadIdx.x & 31) == 0) { s_m[grp] = M; s_l[grp] = L; }
  s_acc[grp][threadIdx.x & 31] = acc;
  __syncthreads();
  if (grp != 0) return;
  float Mt = -INFINITY;
#pragma unroll
  for (int g2 = 0; g2 < 8; ++g2) Mt = fmaxf(Mt, s_m[g2]);
  float Lt = 0.f;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int g2 = 0; g2 < 8; ++g2) {
    if (s_l[g2] == 0.f) continue;
    const float f = __builtin_amdgcn_exp2f(s_m[g2] - Mt);
    const float4 v = s_acc[g2][threadIdx.x & 31];
    Lt += s_l[g2] * f;
    a.x += v.x * f; a.y += v.y * f; a.z += v.z * f; a.w += v.w * f;
  }
  const int b = bh / Hkv, g = bh % Hkv;
  const int tok = r / G, h = g * G + r % G;
  const int Hq = Hkv * G;
  const int64_t m = static_cast<int64_t>(b) * Lq + tok;
  T* dst = tiled ? out + xtile_offset(m, h * kDh + d4, Hq * kDh) : out + (m * Hq + h) * kDh + d4;
  Elem<T>::store(dst, 0, a.x / Lt);
  Elem<T>::store(dst, 1, a.y / Lt);
  Elem<T>::store(dst, 2, a.z / Lt);
  Elem<T>::store(dst, 3, a.w / Lt);
}

// ------------------------------------------------------------- f32 path
// One wave per (packed row, b * Hkv): lane j owns dh elements j and j + 64.
__global__ void attn_f32_kernel(const float* __restrict__ qrot, const float* __restrict__ k_cache,
                                const float* __restrict__ v_cache,
                                const int32_t* __restrict__ prefix_len, int Lq, int G, int Hkv,
                                int Tmax, int dh, int mask_blk, float scale,
                                float* __restrict__ out) {
  const int r = blockIdx.x, bh = blockIdx.y;
  const int b = bh / Hkv, g = bh % Hkv;
  const int lane = threadIdx.x;
  const int rows_total = Lq * G;
  const int tok = r / G;
  const int P = prefix_len[b];
  const int n_keys = min(P + (mask_blk ? attn_block_end(tok, mask_blk, Lq) : Lq), Tmax);   // never past the cache
  const float* qr = qrot + (static_cast<int64_t>(bh) * rows_total + r) * dh;
  const float q0 = lane < dh ? qr[lane] : 0.f;
  const float q1 = lane + 64 < dh ? qr[lane + 64] : 0.f;
  const float* kb = k_cache + static_cast<int64_t>(bh) * Tmax * dh;
  const float* vb = v_cache + static_cast<int64_t>(bh) * Tmax * dh;
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  for (int t = 0; t < n_keys; ++t) {
    const float* kt = kb + static_cast<int64_t>(t) * dh;
    float part = (lane < dh ? q0 * kt[lane] : 0.f) + (lane + 64 < dh ? q1 * kt[lane + 64] : 0.f);
    const float s = warp_sum(part) * scale;
    const float m_new = fmaxf(m, s);
    const float alpha = expf(m - m_new);
    const float p = expf(s - m_new);
    const float* vt = vb + static_cast<int64_t>(t) * dh;
    l = l * alpha + p;
    o0 = o0 * alpha + (lane < dh ? p * vt[lane] : 0.f);
    o1 = o1 * alpha + (lane + 64 < dh ? p * vt[lane + 64] : 0.f);
    m = m_new;
  }
  const int h = g * G + r % G;
  const int Hq = Hkv * G;
  float* o = out + ((static_cast<int64_t>(b) * Lq + tok) * Hq + h) * dh;
  if (lane < dh) o[lane] = o0 / l;
  if (lane + 64 < dh) o[lane + 64] = o1 / l;
}

// ------------------------------------------------------------- launchers
// Group size of the block-causal mask: 0 for the canvas mask (the whole
// block), 1 causal, or the AttnArgs' own mask_blk.
static int attn_mask_blk(const AttnArgs& a) {
  if (a.mask_blk > 0) return a.mask_blk;
  return a.mask_mode == DG_MASK_CAUSAL ? 1 : 0;
}

struct AttnPlan {
  int tiles, nsplit, chunk;
  bool decode;          // attn_decode_kernel (rows <= kDecRows)
  size_t q_bytes, o_bytes, ml_bytes;
};

static AttnPlan plan_attention(int B, int Lq, int Hq, int Hkv, int dh, int Tmax, int dtype) {
  AttnPlan p{};
  const int G = Hq / Hkv;
  const int rows = Lq * G;
  const size_t esz = dtype == DG_BF16 ? 2 : 4;
  p.q_bytes = align_up(static_cast<size_t>(B) * Hkv * rows * dh * esz, 256);
  if (dtype == DG_BF16 && rows <= kDecRows && dh == kDh) {
    p.decode = true;
    p.tiles = 1;
    p.chunk = kDecKeys;
    // a fixed number of splits (the workspace does not grow with the cache),
    // each an even share of the row's keys
    p.nsplit = max(1, min((kDecTargetWgs + B * Hkv - 1) / (B * Hkv), (Tmax + 63) / 64));
    p.o_bytes = align_up(static_cast<size_t>(p.nsplit) * B * Hkv * rows * dh * 4, 256);
    p.ml_bytes = align_up(static_cast<size_t>(p.nsplit) * B * Hkv * rows * sizeof(AttnPartialML), 256);
  } else if (dtype == DG_BF16) {
    p.tiles = (rows + kAttnRows - 1) / kAttnRows;
    const int base = p.tiles * B * Hkv;
    // one workgroup per CU (its LDS): more splits than that only add rounds
    // (a few query rows at 1024 workgroups: 14.2 -> 20.6 us, merge 4.8 -> 9.8)
    const int target = 256;
    int ns = (target + base - 1) / base;
    const int max_ns = (Tmax + kAttnKeys - 1) / kAttnKeys;
    ns = max(1, min(ns, max_ns));
    p.chunk = ((Tmax + ns - 1) / ns + kAttnKeys - 1) / kAttnKeys * kAttnKeys;
    p.nsplit = (Tmax + p.chunk - 1) / p.chunk;
    p.o_bytes = align_up(static_cast<size_t>(p.nsplit) * B * Hkv * rows * dh * 4, 256);
    p.ml_bytes = align_up(static_cast<size_t>(p.nsplit) * B * Hkv * rows * sizeof(AttnPartialML), 256);
  }
  return p;
}

size_t attention_workspace_bytes(int B, int Lq, int Hq, int Hkv, int dh, int Tmax, int dtype) {
  const AttnPlan p = plan_attention(B, Lq, Hq, Hkv, dh, Tmax, dtype);
  return p.q_bytes + p.o_bytes + p.ml_bytes;
}

dg_status launch_attention(const AttnArgs& a, void* ws, hipStream_t stream) {
  const AttnPlan p = plan_attention(a.B, a.Lq, a.Hq, a.Hkv, a.dh, a.Tmax, a.dtype);
  const int G = a.Hq / a.Hkv;
  const int rows = a.Lq * G;
  char* w = static_cast<char*>(ws);
  void* qrot = w;
  if (a.dtype == DG_BF16) {
    if (!a.q_ready) {
      rope_kernel<bf16_t><<<a.B * a.Lq, rope_threads(a.dh), 0, stream>>>(
          static_cast<const bf16_t*>(a.q), static_cast<const bf16_t*>(a.k_new),
          static_cast<const bf16_t*>(a.v_new), a.q_stride, a.kv_stride,
          static_cast<bf16_t*>(qrot), static_cast<bf16_t*>(a.k_cache),
          static_cast<bf16_t*>(a.v_cache), a.prefix_len, a.Lq, a.Hq, a.Hkv, a.dh, a.Tmax,
          a.rope_theta, attn_q_scale(a.dh));
      DG_LAUNCH_CHECK();
    }
    float* o_part = reinterpret_cast<float*>(w + p.q_bytes);
    AttnPartialML* ml = reinterpret_cast<AttnPartialML*>(w + p.q_bytes + p.o_bytes);
    if (p.decode) {
      const unsigned grid = static_cast<unsigned>(p.nsplit) * a.B * a.Hkv;
      if (rows <= 2)
        attn_decode_kernel<2><<<grid, 64 * kDecWaves, 0, stream>>>(
            static_cast<const bf16_t*>(qrot), static_cast<const bf16_t*>(a.k_cache),
            static_cast<const bf16_t*>(a.v_cache), a.prefix_len, a.Lq, G, a.Hkv, a.Tmax,
            p.nsplit, a.B * a.Hkv, attn_mask_blk(a), o_part, ml, a.gate.n_done, a.gate.n,
            a.gate.row_done);
      else
        attn_decode_kernel<4><<<grid, 64 * kDecWaves, 0, stream>>>(
            static_cast<const bf16_t*>(qrot), static_cast<const bf16_t*>(a.k_cache),
            static_cast<const bf16_t*>(a.v_cache), a.prefix_len, a.Lq, G, a.Hkv, a.Tmax,
            p.nsplit, a.B * a.Hkv, attn_mask_blk(a), o_part, ml, a.gate.n_done, a.gate.n,
            a.gate.row_done);
    } else {
      const int total = p.tiles * p.nsplit * a.B * a.Hkv;
      dg_status lst = ensure_lds_limit(reinterpret_cast<const void*>(attn_mfma_kernel),
                                       static_cast<int>(kAttnSmemBytes));
      if (lst != DG_OK) return lst;
      attn_mfma_kernel<<<(total + 7) / 8 * 8, 512, kAttnSmemBytes, stream>>>(
          static_cast<const bf16_t*>(qrot), static_cast<const bf16_t*>(a.k_cache),
          static_cast<const bf16_t*>(a.v_cache), a.prefix_len, a.Lq, G, a.Hkv, a.Tmax, p.chunk,
          p.tiles, p.nsplit, a.B * a.Hkv, attn_mask_blk(a), o_part, ml,
          a.gate.n_done, a.gate.n, a.gate.row_done);
    }
    DG_LAUNCH_CHECK();
    if (p.decode)
      attn_combine_few_kernel<bf16_t><<<a.B * a.Hkv * rows, 256, 0, stream>>>(
          o_part, ml, p.nsplit, a.B * a.Hkv, rows, G, a.Hkv, a.Lq, a.out_tiled,
          static_cast<bf16_t*>(a.out), a.gate.n_done, a.gate.n, a.gate.row_done);
    else
      attn_combine_kernel<bf16_t><<<(a.B * a.Hkv * rows + 7) / 8, 256, 0, stream>>>(
          o_part, ml, p.nsplit, a.B * a.Hkv, rows, G, a.Hkv, a.Lq, a.out_tiled,
          static_cast<bf16_t*>(a.out), a.gate.n_done, a.gate.n, a.gate.row_done);
    DG_LAUNCH_CHECK();
  } else {
    rope_kernel<float><<<a.B * a.Lq, rope_threads(a.dh), 0, stream>>>(
        static_cast<const float*>(a.q), static_cast<const float*>(a.k_new),
        static_cast<const float*>(a.v_new), a.q_stride, a.kv_stride, static_cast<float*>(qrot),
        static_cast<float*>(a.k_cache), static_cast<float*>(a.v_cache), a.prefix_len, a.Lq,
        a.Hq, a.Hkv, a.dh, a.Tmax, a.rope_theta, 1.f);
    DG_LAUNCH_CHECK();
    attn_f32_kernel<<<dim3(rows, a.B * a.Hkv), 64, 0, stream>>>(
        static_cast<const float*>(qrot), static_cast<const float*>(a.k_cache),
        static_cast<const float*>(a.v_cache), a.prefix_len, a.Lq, G, a.Hkv, a.Tmax, a.dh,
        attn_mask_blk(a), static_cast<float>(1.0 / sqrt(static_cast<double>(a.dh))),
        static_cast<float*>(a.out));
    DG_LAUNCH_CHECK();
  }
  return DG_OK;
}

dg_status launch_commit(const void* k_new, const void* v_new, int64_t kv_stride, void* k_cache,
                        void* v_cache, int32_t* prefix_len, int B, int L, int Hkv, int dh,
                        int Tmax, float rope_theta, int dtype, bool advance, hipStream_t stream) {
  if (dtype == DG_BF16)
    rope_kernel<bf16_t><<<B * L, rope_threads(dh), 0, stream>>>(
        nullptr, static_cast<const bf16_t*>(k_new), static_cast<const bf16_t*>(v_new), 0,
        kv_stride, nullptr, static_cast<bf16_t*>(k_cache), static_cast<bf16_t*>(v_cache),
        prefix_len, L, Hkv, Hkv, dh, Tmax, rope_theta, 1.f);
  else
    rope_kernel<float><<<B * L, rope_threads(dh), 0, stream>>>(
        nullptr, static_cast<const float*>(k_new), static_cast<const float*>(v_new), 0,
        kv_stride, nullptr, static_cast<float*>(k_cache), static_cast<float*>(v_cache),
        prefix_len, L, Hkv, Hkv, dh, Tmax, rope_theta, 1.f);
  DG_LAUNCH_CHECK();
  if (advance) return launch_advance_prefix(prefix_len, B, L, stream);
  return DG_OK;
}

dg_status launch_advance_prefix(int32_t* prefix_len, int B, int L, hipStream_t stream) {
  advance_prefix_kernel<<<(B + 63) / 64, 64, 0, stream>>>(prefix_len, B, L);
  DG_LAUNCH_CHECK();
  return DG_OK;
}

}  // namespace dg
