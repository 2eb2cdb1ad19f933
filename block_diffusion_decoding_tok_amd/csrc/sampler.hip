// Canvas sampler: one pass over the [B, L, V] logits.
//
// What is computed (the sampler step of the canvas denoiser; summary of the
// DiffusionGemma technical report, section "DiffusionGemma의 구성", sampler
// settings; developer guide, "Uniform State Diffusion"):
//   z = logits / T_s;  maxprob = 1 / sum_v exp(z_v - max z);
//   entropy = ln Z - sum_v p_v (z_v - max z)  (nats);
//   sample = argmax_v (z_v + g_v), g from Philox stream 0, ties -> lowest v;
//   then the commit / re-noise / stop update per row.
//
// Kernel 1 (partials): grid (nsplit, L, B); a 256-thread workgroup owns one
// vocabulary slice of one position.  Each thread keeps its slice (up to 8
// groups of 8 logits, 16-byte loads, coalesced across the workgroup) in
// registers and walks it three times: max; exp-sum and entropy accumulator
// relative to its own max (float terms, double accumulation); Gumbel-max
// (skipped for a committed position, whose token stays).
// The workgroup merges the per-thread statistics (online-softmax rescaling in
// double) and writes one 32-byte partial.  HBM traffic: the logits once.
//
// Kernel 2 (finish): one workgroup per row merges the nsplit partials of each
// position, computes maxprob / entropy / the row's mean entropy, decides
// whether this step ends the row, and applies the update.
#include <mutex>

#include "common.h"
#include "philox.h"
#include "kernels.h"

namespace dg {

struct SamplerPartial {
  float lmax;        // max raw logit of the slice
  float best_score;  // max of z + g over the slice
  int32_t best_v;    // its id (lowest on ties)
  int32_t flags;     // bit 0: non-finite logit seen
  double Z;          // sum exp((l - lmax) / T)
  double A;          // sum exp((l - lmax) / T) * (l - lmax) / T
};

constexpr int kSampThreads = 256;
constexpr int kSampGroups = 8;                       // groups of 8 logits per thread
constexpr int kSampSlice = kSampThreads * 8 * kSampGroups;   // 16384 logits

template <typename T> struct Vec8;
template <> struct Vec8<bf16_t> {
  uint4 raw;
  __device__ void load(const bf16_t* p) { raw = *reinterpret_cast<const uint4*>(p); }
  __device__ float get(int j) const {
    const uint32_t w = (j < 2) ? raw.x : (j < 4) ? raw.y : (j < 6) ? raw.z : raw.w;
    return (j & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  }
};
template <> struct Vec8<float> {
  float4 a, b;
  __device__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ float get(int j) const {
    switch (j) {
      case 0: return a.x; case 1: return a.y; case 2: return a.z; case 3: return a.w;
      case 4: return b.x; case 5: return b.y; case 6: return b.z; default: return b.w;
    }
  }
};

template <typename T>
__global__ __launch_bounds__(kSampThreads) void sampler_partial_kernel(
    const T* __restrict__ logits, int L, int V, int slice, int nsplit, float invT,
    uint32_t k0, uint32_t k1, int step, const int32_t* __restrict__ prefix_len,
    const int32_t* __restrict__ done, const uint8_t* __restrict__ committed,
    SamplerPartial* __restrict__ part) {
  const int split = blockIdx.x, i = blockIdx.y, b = blockIdx.z;
  if (done[b]) return;
  // a committed position keeps its token: only its maxprob and entropy are
  // needed, so its slices skip the Gumbel draws (workgroup-uniform)
  const bool want_sample = !committed[static_cast<size_t>(b) * L + i];
  const int tid = threadIdx.x;
  const int v_begin = split * slice;
  const int v_end = min(V, v_begin + slice);
  const T* row = logits + (static_cast<size_t>(b) * L + i) * V;

  Vec8<T> vals[kSampGroups];
  bool valid[kSampGroups];
#pragma unroll
  for (int g = 0; g < kSampGroups; ++g) {
    const int v0 = v_begin + (g * kSampThreads + tid) * 8;
    valid[g] = v0 < v_end;
    if (valid[g]) vals[g].load(row + v0);
  }

  // pass 1: max and Gumbel-max over the slice (increasing v per thread)
  const uint32_t pos = static_cast<uint32_t>(prefix_len[b] + i);
  const uint32_t c3 = (kStreamGumbel << 24) | static_cast<uint32_t>(b);
  float lmax = -INFINITY;
  float best = -INFINITY;
  int best_v = 0x7fffffff;
  if (!want_sample) {
#pragma unroll
    for (int g = 0; g < kSampGroups; ++g) {
      if (!valid[g]) continue;
#pragma unroll
      for (int j = 0; j < 8; ++j) lmax = fmaxf(lmax, vals[g].get(j));
    }
  } else {
#pragma unroll
  for (int g = 0; g < kSampGroups; ++g) {
    if (!valid[g]) continue;
    const int v0 = v_begin + (g * kSampThreads + tid) * 8;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const Philox4 r = philox4x32_10(static_cast<uint32_t>((v0 >> 2) + h), pos,
                                      static_cast<uint32_t>(step), c3, k0, k1);
      const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float x = vals[g].get(4 * h + q);
        lmax = fmaxf(lmax, x);
        const float sc = __builtin_fmaf(x, invT, gumbel_from_word(w[q]));
        if (sc > best) { best = sc; best_v = v0 + 4 * h + q; }
      }
    }
  }
  }

  // pass 2: Z and A relative to the thread's own max, in units of log2
  const float log2e = 1.4426950408889634f;
  const float scale2 = invT * log2e;
  double Z = 0.0, A2 = 0.0;
#pragma unroll
  for (int g = 0; g < kSampGroups; ++g) {
    if (!valid[g]) continue;
    float zs = 0.f, as = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float d2 = (vals[g].get(j) - lmax) * scale2;   // <= 0
      const float e = __builtin_amdgcn_exp2f(d2);
      zs += e;
      as = __builtin_fmaf(e, d2, as);
    }
    Z += zs;
    A2 += as;
  }
  // a non-finite logit shows in the sums: NaN propagates through the
  // differences, +inf makes lmax infinite (and inf - inf NaN), -inf gives
  // 0 * -inf = NaN in A
  bool any_valid = false;
#pragma unroll
  for (int g = 0; g < kSampGroups; ++g) any_valid |= valid[g];
  const bool nonfinite = any_valid && !(isfinite(lmax) && isfinite(Z) && isfinite(A2));

  // workgroup merge: max, then rescale (double), then Gumbel best
  __shared__ float s_max[kSampThreads / 64];
  __shared__ double s_Z[kSampThreads / 64], s_A[kSampThreads / 64];
  __shared__ float s_best[kSampThreads / 64];
  __shared__ int s_bv[kSampThreads / 64], s_nf[kSampThreads / 64];
  const int lane = tid & 63, wv = tid >> 6;
  float m = warp_max(lmax);
  if (lane == 0) s_max[wv] = m;
  __syncthreads();
  float M = s_max[0];
#pragma unroll
  for (int w2 = 1; w2 < kSampThreads / 64; ++w2) M = fmaxf(M, s_max[w2]);
  double Zt = 0.0, At = 0.0;
  if (Z > 0.0) {
    // rescale this thread's sums from its max to the slice max: factor
    // exp(delta), delta = (lmax - M) / T; A_nat = ln2 * A2 + delta * Z
    const double delta = static_cast<double>(lmax - M) * static_cast<double>(invT);
    const double f = exp(delta);
    Zt = Z * f;
    At = f * (A2 * 0.69314718055994530942 + delta * Z);
  }
  Zt = warp_sum_d(Zt);
  At = warp_sum_d(At);
  // best: max score, lowest id on ties
  for (int o = 32; o > 0; o >>= 1) {
    const float ob = __shfl_xor(best, o);
    const int ov = __shfl_xor(best_v, o);
    if (ob > best || (ob == best && ov < best_v)) { best = ob; best_v = ov; }
  }
  const int nf = __any(nonfinite) ? 1 : 0;
  if (lane == 0) { s_Z[wv] = Zt; s_A[wv] = At; s_best[wv] = best; s_bv[wv] = best_v; s_nf[wv] = nf; }
  __syncthreads();
  if (tid == 0) {
    SamplerPartial p;
    p.lmax = M;
    p.Z = 0.0; p.A = 0.0;
    p.best_score = -INFINITY; p.best_v = 0x7fffffff; p.flags = 0;
    for (int w2 = 0; w2 < kSampThreads / 64; ++w2) {
      p.Z += s_Z[w2];
      p.A += s_A[w2];
      if (s_best[w2] > p.best_score || (s_best[w2] == p.best_score && s_bv[w2] < p.best_v)) {
        p.best_score = s_best[w2];
        p.best_v = s_bv[w2];
      }
      p.flags |= s_nf[w2];
    }
    part[(static_cast<size_t>(b) * L + i) * nsplit + split] = p;
  }
}

constexpr int kFinishThreads = 1024;

// One workgroup per row.  Merge: 16 lanes per position (lane sl takes
// splits sl, sl + 16, ...), shuffle reductions in a fixed order.  The
// entropy-bound ranking sorts (entropy, position) keys with a bitonic sort in
// LDS (committed positions and the padding up to npow2 take +inf), then each
// thread walks a contiguous segment of the sorted keys with its exclusive
// prefix sum (segment sums scanned across the workgroup).
__global__ __launch_bounds__(kFinishThreads) void sampler_finish_kernel(
    const SamplerPartial* __restrict__ part, int L, int npow2, int V, int nsplit, float invT,
    int step, int ends_at_step, int adaptive, float stop_entropy, float commit_prob,
    float renoise_prob, int policy, float entropy_bound, uint32_t k0, uint32_t k1,
    const int32_t* __restrict__ prefix_len,
    int32_t* __restrict__ tokens, uint8_t* __restrict__ committed,
    uint8_t* __restrict__ renoised, float* __restrict__ maxprob, float* __restrict__ entropy,
    float* __restrict__ mean_entropy, int32_t* __restrict__ done, int32_t* __restrict__ status,
    int32_t* __restrict__ steps_taken, int32_t* __restrict__ n_done) {
  const int b = blockIdx.x;
  if (done[b]) return;
  const int tid = threadIdx.x;
  extern __shared__ unsigned char smem_raw[];
  double* s_mp = reinterpret_cast<double*>(smem_raw);           // [L]
  double* s_key = s_mp + L;                                     // [npow2] entropies
  int32_t* s_sample = reinterpret_cast<int32_t*>(s_key + npow2);   // [L]
  int32_t* s_idx = s_sample + L;                                // [npow2]
  uint8_t* s_flag = reinterpret_cast<uint8_t*>(s_idx + npow2);  // [L] bit 0: uncommitted
  constexpr int kWaves = kFinishThreads / 64;
  __shared__ double s_red[kWaves];
  __shared__ int s_nf[kWaves];

  // ---- per-position merge of the slice partials
  const int sl = tid & 15, grp = tid >> 4;
  constexpr int kGroups = kFinishThreads / 16;
  double hsum = 0.0;
  int nf = 0;
  for (int i0 = 0; i0 < L; i0 += kGroups) {
    const int i = i0 + grp;
    const bool act = i < L;                      // uniform in the 16-lane group
    const SamplerPartial* p = part + (static_cast<size_t>(b) * L + (act ? i : 0)) * nsplit;
    float M = -INFINITY;
    for (int s = sl; s < nsplit; s += 16) M = fmaxf(M, p[s].lmax);
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    double Z = 0.0, A = 0.0;
    float best = -INFINITY;
    int best_v = 0x7fffffff;
    for (int s = sl; s < nsplit; s += 16) {
      const SamplerPartial q = p[s];
      nf |= q.flags;
      if (q.Z > 0.0) {
        const double delta = static_cast<double>(q.lmax - M) * static_cast<double>(invT);
        const double f = exp(delta);
        Z += q.Z * f;
        A += f * (q.A + delta * q.Z);
      }
      if (q.best_score > best || (q.best_score == best && q.best_v < best_v)) {
        best = q.best_score;
        best_v = q.best_v;
      }
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) {
      Z += __shfl_xor(Z, o);
      A += __shfl_xor(A, o);
      const float ob = __shfl_xor(best, o);
      const int ov = __shfl_xor(best_v, o);
      if (ob > best || (ob == best && ov < best_v)) { best = ob; best_v = ov; }
    }
    if (act && sl == 0) {
      const double mp = 1.0 / Z;
      const double H = log(Z) - A / Z;
      s_mp[i] = mp;
      s_key[i] = H;
      s_sample[i] = best_v;
      s_flag[i] = committed[static_cast<size_t>(b) * L + i] ? 0 : 1;
      maxprob[static_cast<size_t>(b) * L + i] = static_cast<float>(mp);
      entropy[static_cast<size_t>(b) * L + i] = static_cast<float>(H);
      hsum += H;
    }
  }
  hsum = warp_sum_d(hsum);
  nf = __any(nf) ? 1 : 0;
  if ((tid & 63) == 0) { s_red[tid >> 6] = hsum; s_nf[tid >> 6] = nf; }
  __syncthreads();
  double tot = 0.0;
  int anynf = 0;
  for (int w = 0; w < kWaves; ++w) { tot += s_red[w]; anynf |= s_nf[w]; }
  const double hbar = tot / L;

  // ---- entropy-bound policy: an uncommitted position commits when the
  // entropies of the uncommitted positions ranked below it, by (entropy,
  // position), sum to at most the bound (the longest ranked prefix whose sum
  // minus its largest term is within the bound)
  bool all_committed = false;
  if (policy == DG_COMMIT_ENTROPY_BOUND) {
    for (int r = tid; r < npow2; r += kFinishThreads) {
      if (!(r < L && (s_flag[r] & 1))) s_key[r] = INFINITY;
      s_idx[r] = r;
    }
    __syncthreads();
    for (int k = 2; k <= npow2; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int t = tid; t < npow2; t += kFinishThreads) {
          const int u = t ^ j;
          if (u > t) {
            const double ka = s_key[t], kb = s_key[u];
            const int ia = s_idx[t], ib = s_idx[u];
            const bool a_after = ka > kb || (ka == kb && ia > ib);
            if (a_after == ((t & k) == 0)) {       // ascending runs where (t & k) == 0
              s_key[t] = kb; s_key[u] = ka;
              s_idx[t] = ib; s_idx[u] = ia;
            }
          }
        }
        __syncthreads();
      }
    }
    // exclusive prefix sums of the sorted finite keys: thread segments of
    // seg keys, segment totals scanned through the waves
    const int seg = (npow2 + kFinishThreads - 1) / kFinishThreads;
    const int r0 = min(tid * seg, npow2), r1 = min(r0 + seg, npow2);
    double part_sum = 0.0;
    for (int r = r0; r < r1; ++r) {
      const double kv = s_key[r];
      if (kv < INFINITY) part_sum += kv;
    }
    const int lane = tid & 63, wv = tid >> 6;
    double incl = part_sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const double t2 = __shfl_up(incl, o);
      if (lane >= o) incl += t2;
    }
    __syncthreads();                     // s_red reused for the wave totals
    if (lane == 63) s_red[wv] = incl;
    __syncthreads();
    double run = incl - part_sum;
    for (int w = 0; w < wv; ++w) run += s_red[w];
    int left = 0;                        // uncommitted positions that stay so
    for (int r = r0; r < r1; ++r) {
      const double kv = s_key[r];
      if (!(kv < INFINITY)) continue;
      if (run <= static_cast<double>(entropy_bound)) s_flag[s_idx[r]] |= 2;
      else left = 1;
      run += kv;
    }
    all_committed = __syncthreads_or(left) == 0;
  }
  const bool ends = adaptive ? (hbar < static_cast<double>(stop_entropy) || step == ends_at_step ||
                                all_committed)
                             : (step == ends_at_step);
  if (tid == 0) {
    mean_entropy[b] = static_cast<float>(hbar);
    done[b] = ends ? 1 : 0;
    if (ends && n_done) atomicAdd(n_done, 1);
    if (steps_taken) steps_taken[b] += 1;
    if (anynf && status) atomicOr(status, DG_STATUS_NONFINITE_LOGITS);
  }
  __syncthreads();                       // s_flag complete before the update
  const uint32_t c3r = (kStreamRenoise << 24) | static_cast<uint32_t>(b);
  for (int i = tid; i < L; i += kFinishThreads) {
    const size_t o = static_cast<size_t>(b) * L + i;
    uint8_t ren = 0;
    if (!committed[o]) {
      const double mpd = s_mp[i];   // thresholds compared in double
      const bool commit = policy == DG_COMMIT_ENTROPY_BOUND
                              ? (s_flag[i] & 2) != 0
                              : mpd >= static_cast<double>(commit_prob);
      if (commit) {
        tokens[o] = s_sample[i];
        committed[o] = 1;
      } else if (mpd < static_cast<double>(renoise_prob) && !ends) {
        const uint32_t pos = static_cast<uint32_t>(prefix_len[b] + i);
        const Philox4 r = philox4x32_10(0u, pos, static_cast<uint32_t>(step), c3r, k0, k1);
        tokens[o] = static_cast<int32_t>(uniform_id(r.x, static_cast<uint32_t>(V)));
        ren = 1;
      } else {
        tokens[o] = s_sample[i];
      }
    }
    renoised[o] = ren;
  }
}

dg_status launch_sampler(const void* logits, int logit_dtype, int B, int L, int V, int step,
                         const dg_sampler_cfg& cfg, const int32_t* prefix_len, int32_t* tokens,
                         uint8_t* committed, uint8_t* renoised, float* maxprob, float* entropy,
                         float* mean_entropy, int32_t* done, int32_t* status,
                         int32_t* steps_taken, void* ws, hipStream_t stream, int32_t* n_done) {
  const int nsplit = (V + kSampSlice - 1) / kSampSlice;
  const int slice = ((V + nsplit - 1) / nsplit + 7) / 8 * 8;
  const int S = cfg.max_steps;
  const double T = (S <= 1) ? cfg.temp_start
                            : cfg.temp_start + (static_cast<double>(cfg.temp_end) - cfg.temp_start) *
                                                   step / (S - 1);
  const float invT = static_cast<float>(1.0 / T);
  const uint32_t k0 = static_cast<uint32_t>(cfg.seed), k1 = static_cast<uint32_t>(cfg.seed >> 32);
  SamplerPartial* part = reinterpret_cast<SamplerPartial*>(ws);
  dim3 grid(nsplit, L, B);
  if (logit_dtype == DG_BF16)
    sampler_partial_kernel<bf16_t><<<grid, kSampThreads, 0, stream>>>(
        static_cast<const bf16_t*>(logits), L, V, slice, nsplit, invT, k0, k1, step, prefix_len,
        done, committed, part);
  else
    sampler_partial_kernel<float><<<grid, kSampThreads, 0, stream>>>(
        static_cast<const float*>(logits), L, V, slice, nsplit, invT, k0, k1, step, prefix_len,
        done, committed, part);
  DG_LAUNCH_CHECK();
  const int adaptive = cfg.fixed_steps > 0 ? 0 : 1;
  const int ends_at = cfg.fixed_steps > 0 ? cfg.fixed_steps - 1 : S - 1;
  int npow2 = 1;
  while (npow2 < L) npow2 <<= 1;
  const size_t smem = static_cast<size_t>(L) * (sizeof(double) + sizeof(int32_t) + 1) +
                      static_cast<size_t>(npow2) * (sizeof(double) + sizeof(int32_t));
  // up to 4096 positions: 100 KB of LDS
  const dg_status lst =
      ensure_lds_limit(reinterpret_cast<const void*>(sampler_finish_kernel), 4096 * 25);
  if (lst != DG_OK) return lst;
  sampler_finish_kernel<<<B, kFinishThreads, smem, stream>>>(
      part, L, npow2, V, nsplit, invT, step, ends_at, adaptive, cfg.stop_entropy, cfg.commit_prob,
      cfg.renoise_prob, cfg.commit_policy, cfg.entropy_bound, k0, k1, prefix_len, tokens,
      committed, renoised, maxprob, entropy, mean_entropy, done, status, steps_taken, n_done);
  DG_LAUNCH_CHECK();
  return DG_OK;
}

size_t sampler_workspace_bytes(int B, int L, int V) {
  const int nsplit = (V + kSampSlice - 1) / kSampSlice;
  return align_up(static_cast<size_t>(B) * L * nsplit * sizeof(SamplerPartial), 256);
}

// ------------------------------------------------- library-owned scratch
// The workspace of dg_sampler_step_noalloc: one array per GPU the library
// runs on, held until the process ends.  Host code never uses the array's
// name as an address: the device address comes from hipGetSymbolAddress,
// taken once per device with that device current.
constexpr size_t kSamplerScratchBytes = size_t(1) << 20;
static_assert(kSamplerScratchBytes == DG_SAMPLER_SCRATCH_BYTES, "scratch size");
static __device__ __align__(256) unsigned char scratch[kSamplerScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array.
static dg_status scratch_ptr(void** out) {
  int dev = 0;
  DG_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(DG_ERR_UNSUPPORTED, "device index out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    DG_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(DG_ERR_HIP, "hipGetSymbolAddress returned a null scratch address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DG_OK;
}

// ------------------------------------------------------------ init canvas
__global__ void init_canvas_kernel(const int32_t* __restrict__ prefix_len, int B, int L, int V,
                                   uint32_t k0, uint32_t k1, int32_t* __restrict__ tokens,
                                   uint8_t* __restrict__ committed, int32_t* __restrict__ done) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx < B) done[idx] = 0;
  if (idx >= B * L) return;
  const int b = idx / L, i = idx % L;
  const uint32_t pos = static_cast<uint32_t>(prefix_len[b] + i);
  const Philox4 r = philox4x32_10(0u, pos, 0u, (kStreamCanvas << 24) | static_cast<uint32_t>(b), k0, k1);
  tokens[idx] = static_cast<int32_t>(uniform_id(r.x, static_cast<uint32_t>(V)));
  committed[idx] = 0;
}

dg_status launch_init_canvas(const int32_t* prefix_len, int B, int L, int V, uint64_t seed,
                             int32_t* tokens, uint8_t* committed, int32_t* done,
                             hipStream_t stream) {
  const int n = max(B * L, B);
  init_canvas_kernel<<<(n + 255) / 256, 256, 0, stream>>>(
      prefix_len, B, L, V, static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32), tokens,
      committed, done);
  DG_LAUNCH_CHECK();
  return DG_OK;
}

// ------------------------------------------------------------ test hooks
__global__ void philox_kernel(const uint32_t* __restrict__ ctr, int64_t n, uint32_t k0,
                              uint32_t k1, uint32_t* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const Philox4 r = philox4x32_10(ctr[4 * i], ctr[4 * i + 1], ctr[4 * i + 2], ctr[4 * i + 3], k0, k1);
  out[4 * i] = r.x; out[4 * i + 1] = r.y; out[4 * i + 2] = r.z; out[4 * i + 3] = r.w;
}

__global__ void gumbel_kernel(const uint32_t* __restrict__ w, int64_t n, float* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) out[i] = gumbel_from_word(w[i]);
}

dg_status launch_philox(const uint32_t* ctr, int64_t n, uint64_t seed, uint32_t* out,
                        hipStream_t stream) {
  if (n == 0) return DG_OK;
  philox_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, stream>>>(
      ctr, n, static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32), out);
  DG_LAUNCH_CHECK();
  return DG_OK;
}

dg_status launch_gumbel(const uint32_t* w, int64_t n, float* out, hipStream_t stream) {
  if (n == 0) return DG_OK;
  gumbel_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, stream>>>(w, n, out);
  DG_LAUNCH_CHECK();
  return DG_OK;
}

}  // namespace dg

extern "C" dg_status dg_sampler_step_noalloc(const void* logits, int logit_dtype, int B, int L,
                                             int V, int step, const dg_sampler_cfg* cfg,
                                             const int32_t* prefix_len, int32_t* tokens,
                                             uint8_t* committed, uint8_t* renoised,
                                             float* maxprob, float* entropy, float* mean_entropy,
                                             int32_t* done, int32_t* status, void* stream) {
  using namespace dg;
  set_error("");
  dg_status st = check_sampler_step(logits, logit_dtype, B, L, V, step, cfg, prefix_len, tokens,
                                    committed, renoised, maxprob, entropy, mean_entropy, done);
  if (st != DG_OK) return st;
  if (sampler_workspace_bytes(B, L, V) > kSamplerScratchBytes)
    return fail(DG_ERR_WORKSPACE,
                "dg_sampler_step_noalloc: B * L * ceil(V / 16384) * 32 bytes exceed the "
                "library's 1 MiB scratch");
  void* ws = nullptr;
  if ((st = scratch_ptr(&ws))) return st;
  // every partial the finishing kernel reads is written earlier in the same
  // call, so the scratch needs no clearing
  return launch_sampler(logits, logit_dtype, B, L, V, step, *cfg, prefix_len, tokens, committed,
                        renoised, maxprob, entropy, mean_entropy, done, status, nullptr, ws,
                        static_cast<hipStream_t>(stream));
}
