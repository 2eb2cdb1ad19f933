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
//   1. rope_kernel: per token (heads spread over the workgroup's threads),
//      rotates the block's q (into a packed workspace
//      [B, Hkv, Lq * G, dh], packed row r = token * G + (head % G)) and k
//      (into cache slots [P, P + Lq)), copies v into the cache.
//   2. bf16: attn_mfma_kernel, grid (row tiles of 128, KV splits, B * Hkv);
//      four waves x 32 packed rows; K tile [64 keys][dh] and V^T tile
//      [dh][64 keys] staged in LDS (double buffered); S^T = K Q^T and
//      O^T = V^T P^T on v_mfma_f32_16x16x32_bf16 so that the probabilities
//      leave the S MFMA already in the B-operand layout of the PV MFMA.
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
    int dh, int Tmax, float theta) {
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
      Elem<T>::store(dst, j, x1 * c - x2 * s);
      Elem<T>::store(dst, j + half, x2 * c + x1 * s);
    }
  }
  const T* kt = k_new + static_cast<int64_t>(tok) * kv_stride;
  const T* vt = v_new + static_cast<int64_t>(tok) * kv_stride;
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
constexpr int kAttnRows = 128;        // packed rows per workgroup
constexpr int kAttnKeys = 64;         // keys per LDS tile
constexpr int kDh = 128;
constexpr int kKStride = kDh + 8;     // K tile row stride (elements): 272 B
constexpr int kVStride = kAttnKeys + 8;   // V^T tile row stride: 144 B
constexpr int kKTileElems = kAttnKeys * kKStride;
constexpr int kVTileElems = kDh * kVStride;

// Column of key kappa (0..63) in a V^T tile row: within each 32-key chunk the
// keys are placed so that the 8 keys a lane feeds to one PV MFMA (4 from each
// 16-key block, matching the S^T accumulator layout) are contiguous.
__device__ __forceinline__ int vt_col(int kappa) {
  const int t = kappa >> 5, w = kappa & 31;
  return t * 32 + ((w & 15) >> 2) * 8 + ((w >> 4) << 2) + (w & 3);
}

struct AttnPartialML { float m, l; };

__global__ __launch_bounds__(256) void attn_mfma_kernel(
    const bf16_t* __restrict__ qrot, const bf16_t* __restrict__ k_cache,
    const bf16_t* __restrict__ v_cache, const int32_t* __restrict__ prefix_len, int Lq, int G,
    int Hkv, int Tmax, int chunk, int nsplit, int causal, float scale_log2,
    float* __restrict__ o_part, AttnPartialML* __restrict__ ml_part) {
  __shared__ __attribute__((aligned(16))) bf16_t s_k[2][kKTileElems];
  __shared__ __attribute__((aligned(16))) bf16_t s_v[2][kVTileElems];

  const int tile = blockIdx.x, split = blockIdx.y, bh = blockIdx.z;
  const int b = bh / Hkv;
  const int rows_total = Lq * G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int P = prefix_len[b];
  const int n_keys = P + Lq;
  const int row0 = tile * kAttnRows + wave * 32;   // this wave's first packed row

  // key range of this split (causal: trimmed to the last row of the tile)
  int k_begin = split * chunk;
  int k_end = min(n_keys, k_begin + chunk);
  if (causal) {
    const int last_row = min(rows_total - 1, tile * kAttnRows + kAttnRows - 1);
    k_end = min(k_end, P + last_row / G + 1);
  }
  const int ntiles = k_end > k_begin ? (k_end - k_begin + kAttnKeys - 1) / kAttnKeys : 0;

  // Q fragments (B operand of S^T = K Q^T): row l16 of each 16-row block,
  // dh 32c + 8 g4 .. +7
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
  // token of each of this lane's two rows (for the causal mask)
  int tok_of[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) tok_of[qb] = (row0 + qb * 16 + l16) / G;

  f32x4_t acc_o[2][8];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int d = 0; d < 8; ++d) acc_o[qb][d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};

  const bf16_t* kbase = k_cache + static_cast<int64_t>(bh) * Tmax * kDh;
  const bf16_t* vbase = v_cache + static_cast<int64_t>(bh) * Tmax * kDh;

  // staging: K tile = 64 keys x 16 chunks of 8 dh (1024 items of 16 B, four
  // per thread); V tile = 16 quads of 4 keys x 16 chunks of 8 dh (one item
  // of 4 x 16 B per thread), written transposed into V^T.
  uint4 kreg[4];
  uint4 vreg[4];
  auto load_tile = [&](int t) {
    const int key0 = k_begin + t * kAttnKeys;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int item = it * 256 + tid;
      const int key = item >> 4, ch = item & 15;
      const int gk = key0 + key;
      kreg[it] = (gk < k_end) ? *reinterpret_cast<const uint4*>(kbase + static_cast<int64_t>(gk) * kDh + ch * 8)
                              : make_uint4(0, 0, 0, 0);
    }
    {
      const int kq = tid >> 4, ch = tid & 15;     // 4-key quad kq (0..15), dh chunk ch
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int gk = key0 + kq * 4 + kk;
        vreg[kk] = (gk < k_end) ? *reinterpret_cast<const uint4*>(vbase + static_cast<int64_t>(gk) * kDh + ch * 8)
                                : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int item = it * 256 + tid;
      const int key = item >> 4, ch = item & 15;
      *reinterpret_cast<uint4*>(&s_k[buf][key * kKStride + ch * 8]) = kreg[it];
    }
    const int kq = tid >> 4, ch = tid & 15;
    const int col = vt_col(kq * 4);   // 4 consecutive keys -> 4 consecutive columns
    const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&vreg[0]);
    const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&vreg[1]);
    const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vreg[2]);
    const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&vreg[3]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sh = (e & 1) * 16;
      const uint32_t a0 = (w0[e >> 1] >> sh) & 0xffffu, a1 = (w1[e >> 1] >> sh) & 0xffffu;
      const uint32_t a2 = (w2[e >> 1] >> sh) & 0xffffu, a3 = (w3[e >> 1] >> sh) & 0xffffu;
      uint2 pk;
      pk.x = a0 | (a1 << 16);
      pk.y = a2 | (a3 << 16);
      *reinterpret_cast<uint2*>(&s_v[buf][(ch * 8 + e) * kVStride + col]) = pk;
    }
  };

  if (ntiles > 0) load_tile(0);
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    store_tile(buf);
    __syncthreads();
    if (t + 1 < ntiles) load_tile(t + 1);
    const int key0 = k_begin + t * kAttnKeys;

    // S^T blocks: [kb][qb], keys kb*16 + 4 g4 + r, row l16
    f32x4_t s_acc[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) s_acc[kb][qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(
            &s_k[buf][(kb * 16 + l16) * kKStride + c * 32 + g4 * 8]);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          s_acc[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[qb][c], s_acc[kb][qb], 0, 0, 0);
      }
    }
    // mask, online softmax (log2 domain), probabilities -> bf16 B operands
    bf16x8_t pf[2][2];   // [qb][32-key chunk]
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int key_lim = causal ? min(k_end, P + tok_of[qb] + 1) : k_end;
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = key0 + kb * 16 + g4 * 4 + r;
          float v = s_acc[kb][qb][r] * scale_log2;
          v = (key < key_lim) ? v : -INFINITY;
          s_acc[kb][qb][r] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[qb], mx);
      const float base = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - base);
      m_run[qb] = m_new;
      float rs = 0.f;
      uint32_t pk[2][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[r] = __builtin_amdgcn_exp2f(s_acc[kb][qb][r] - base);
          rs += p[r];
        }
        pk[kb >> 1][(kb & 1) * 2 + 0] = pack_bf16x2(p[0], p[1]);
        pk[kb >> 1][(kb & 1) * 2 + 1] = pack_bf16x2(p[2], p[3]);
      }
      l_run[qb] = l_run[qb] * alpha + rs;
#pragma unroll
      for (int d = 0; d < 8; ++d) acc_o[qb][d] *= alpha;
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
        uint4 u = make_uint4(pk[ch][0], pk[ch][1], pk[ch][2], pk[ch][3]);
        pf[qb][ch] = *reinterpret_cast<bf16x8_t*>(&u);
      }
    }
    // O^T[d] += V^T[d block] P^T
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const bf16x8_t va = *reinterpret_cast<const bf16x8_t*>(
            &s_v[buf][(d * 16 + l16) * kVStride + ch * 32 + g4 * 8]);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          acc_o[qb][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pf[qb][ch], acc_o[qb][d], 0, 0, 0);
      }
    }
  }

  // write the split's partial: O unnormalized [rows][dh] f32, (m, l) per row
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float l = l_run[qb];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int r = row0 + qb * 16 + l16;
    if (r >= rows_total) continue;
    const int64_t prow = (static_cast<int64_t>(split) * gridDim.z + bh) * rows_total + r;
    float* dst = o_part + prow * kDh;
#pragma unroll
    for (int d = 0; d < 8; ++d)
      *reinterpret_cast<float4*>(dst + d * 16 + g4 * 4) =
          make_float4(acc_o[qb][d][0], acc_o[qb][d][1], acc_o[qb][d][2], acc_o[qb][d][3]);
    if (g4 == 0) ml_part[prow] = AttnPartialML{m_run[qb], l};
  }
}

// Merge the KV splits of every packed row and write out [B, Lq, Hq, dh].
template <typename T>
__global__ void attn_combine_kernel(const float* __restrict__ o_part,
                                    const AttnPartialML* __restrict__ ml_part, int nsplit,
                                    int BH, int rows_total, int G, int Hkv, int Lq, int dh,
                                    T* __restrict__ out) {
  const int r = blockIdx.x, bh = blockIdx.y;
  const int d = threadIdx.x;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s)
    M = fmaxf(M, ml_part[(static_cast<int64_t>(s) * BH + bh) * rows_total + r].m);
  const float base = (M == -INFINITY) ? 0.f : M;
  float L = 0.f, acc = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const int64_t prow = (static_cast<int64_t>(s) * BH + bh) * rows_total + r;
    const AttnPartialML ml = ml_part[prow];
    if (ml.l == 0.f) continue;
    const float f = __builtin_amdgcn_exp2f(ml.m - base);
    L += ml.l * f;
    if (d < dh) acc += o_part[prow * dh + d] * f;
  }
  if (d >= dh) return;
  const int b = bh / Hkv, g = bh % Hkv;
  const int tok = r / G, h = g * G + r % G;
  const int Hq = Hkv * G;
  Elem<T>::store(out, ((static_cast<int64_t>(b) * Lq + tok) * Hq + h) * dh + d, acc / L);
}

// ------------------------------------------------------------- f32 path
// One wave per (packed row, b * Hkv): lane j owns dh elements j and j + 64.
__global__ void attn_f32_kernel(const float* __restrict__ qrot, const float* __restrict__ k_cache,
                                const float* __restrict__ v_cache,
                                const int32_t* __restrict__ prefix_len, int Lq, int G, int Hkv,
                                int Tmax, int dh, int causal, float scale,
                                float* __restrict__ out) {
  const int r = blockIdx.x, bh = blockIdx.y;
  const int b = bh / Hkv, g = bh % Hkv;
  const int lane = threadIdx.x;
  const int rows_total = Lq * G;
  const int tok = r / G;
  const int P = prefix_len[b];
  const int n_keys = causal ? P + tok + 1 : P + Lq;
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
struct AttnPlan {
  int tiles, nsplit, chunk;
  size_t q_bytes, o_bytes, ml_bytes;
};

static AttnPlan plan_attention(int B, int Lq, int Hq, int Hkv, int dh, int Tmax, int dtype) {
  AttnPlan p{};
  const int G = Hq / Hkv;
  const int rows = Lq * G;
  const size_t esz = dtype == DG_BF16 ? 2 : 4;
  p.q_bytes = align_up(static_cast<size_t>(B) * Hkv * rows * dh * esz, 256);
  if (dtype == DG_BF16) {
    p.tiles = (rows + kAttnRows - 1) / kAttnRows;
    const int base = p.tiles * B * Hkv;
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
    rope_kernel<bf16_t><<<a.B * a.Lq, rope_threads(a.dh), 0, stream>>>(
        static_cast<const bf16_t*>(a.q), static_cast<const bf16_t*>(a.k_new),
        static_cast<const bf16_t*>(a.v_new), a.q_stride, a.kv_stride,
        static_cast<bf16_t*>(qrot), static_cast<bf16_t*>(a.k_cache),
        static_cast<bf16_t*>(a.v_cache), a.prefix_len, a.Lq, a.Hq, a.Hkv, a.dh, a.Tmax,
        a.rope_theta);
    DG_LAUNCH_CHECK();
    float* o_part = reinterpret_cast<float*>(w + p.q_bytes);
    AttnPartialML* ml = reinterpret_cast<AttnPartialML*>(w + p.q_bytes + p.o_bytes);
    const float scale_log2 = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(a.dh)));
    dim3 grid(p.tiles, p.nsplit, a.B * a.Hkv);
    attn_mfma_kernel<<<grid, 256, 0, stream>>>(
        static_cast<const bf16_t*>(qrot), static_cast<const bf16_t*>(a.k_cache),
        static_cast<const bf16_t*>(a.v_cache), a.prefix_len, a.Lq, G, a.Hkv, a.Tmax, p.chunk,
        p.nsplit, a.mask_mode == DG_MASK_CAUSAL, scale_log2, o_part, ml);
    DG_LAUNCH_CHECK();
    attn_combine_kernel<bf16_t><<<dim3(rows, a.B * a.Hkv), 128, 0, stream>>>(
        o_part, ml, p.nsplit, a.B * a.Hkv, rows, G, a.Hkv, a.Lq, a.dh,
        static_cast<bf16_t*>(a.out));
    DG_LAUNCH_CHECK();
  } else {
    rope_kernel<float><<<a.B * a.Lq, rope_threads(a.dh), 0, stream>>>(
        static_cast<const float*>(a.q), static_cast<const float*>(a.k_new),
        static_cast<const float*>(a.v_new), a.q_stride, a.kv_stride, static_cast<float*>(qrot),
        static_cast<float*>(a.k_cache), static_cast<float*>(a.v_cache), a.prefix_len, a.Lq,
        a.Hq, a.Hkv, a.dh, a.Tmax, a.rope_theta);
    DG_LAUNCH_CHECK();
    attn_f32_kernel<<<dim3(rows, a.B * a.Hkv), 64, 0, stream>>>(
        static_cast<const float*>(qrot), static_cast<const float*>(a.k_cache),
        static_cast<const float*>(a.v_cache), a.prefix_len, a.Lq, G, a.Hkv, a.Tmax, a.dh,
        a.mask_mode == DG_MASK_CAUSAL, static_cast<float>(1.0 / sqrt(static_cast<double>(a.dh))),
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
        prefix_len, L, Hkv, Hkv, dh, Tmax, rope_theta);
  else
    rope_kernel<float><<<B * L, rope_threads(dh), 0, stream>>>(
        nullptr, static_cast<const float*>(k_new), static_cast<const float*>(v_new), 0,
        kv_stride, nullptr, static_cast<float*>(k_cache), static_cast<float*>(v_cache),
        prefix_len, L, Hkv, Hkv, dh, Tmax, rope_theta);
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
