// Shared device/host helpers of libdg (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string>

#include "../../include/dg.h"

namespace dg {

// ------------------------------------------------------------ error state
void set_error(const std::string& msg);
dg_status fail(dg_status st, const std::string& msg);

#define DG_CHECK_ARG(cond, msg) \
  do { if (!(cond)) return ::dg::fail(DG_ERR_INVALID_ARG, msg); } while (0)
#define DG_CHECK_SHAPE(cond, msg) \
  do { if (!(cond)) return ::dg::fail(DG_ERR_SHAPE, msg); } while (0)
#define DG_HIP(call)                                                              \
  do {                                                                            \
    hipError_t e_ = (call);                                                       \
    if (e_ != hipSuccess)                                                         \
      return ::dg::fail(DG_ERR_HIP, std::string(#call) + ": " + hipGetErrorString(e_)); \
  } while (0)
#define DG_LAUNCH_CHECK() DG_HIP(hipGetLastError())

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Raises a kernel's dynamic LDS limit to bytes on the current device, once
// per (kernel, device); safe to call from several threads.
dg_status ensure_lds_limit(const void* kernel, int bytes);

// The tiled activation layout of a bf16 matrix [M, K] (K % 64 == 0) that the
// dense projections can read: one 2 KB block per 16 tokens x 64 k, blocks in
// (token block, k block) order, and inside a block the operand lane order of
// the 16x16x32 MFMA: element (m, k) at (k / 8 % 2) * 512 + ((k / 16 % 4) * 16
// + m % 16) * 8 + k % 8.  Four consecutive k from a multiple of 4 stay
// contiguous.  Storage: ceil(M / 16) * 16 * K elements; rows past M in the
// last block are never written and never used.
__host__ __device__ inline int64_t xtile_offset(int64_t m, int k, int K) {
  const int kk = k & 63;
  return ((m >> 4) * (K >> 6) + (k >> 6)) * 1024 + ((kk >> 3) & 1) * 512 +
         ((kk >> 4) * 16 + (m & 15)) * 8 + (kk & 7);
}

// ------------------------------------------------------------ bf16 helpers
typedef uint16_t bf16_t;   // raw bits

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
// Round-to-nearest-even float -> bf16 with the hardware pair conversion
// (v_cvt_pk_bf16_f32).  Over all 2^32 inputs it equals the integer rule
// u + 0x7fff + ((u >> 16) & 1) >> 16 for non-NaN u, and (u >> 16) | 0x40 for
// NaN (quieted, payload kept), denormals included.
typedef float f32x2_cvt_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_cvt_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_cvt_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_cvt_t));
}
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

// Element loads/stores for the two activation types.
template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static float load(const float* p, size_t i) { return p[i]; }
  __device__ static void store(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<bf16_t> {
  __device__ static float load(const bf16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  __device__ static void store(bf16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
};

// ------------------------------------------------------------ reductions
__device__ __forceinline__ float warp_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float warp_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ double warp_sum_d(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// All-reduce over each 16-lane row of (value, index) pairs: the largest
// value, the lowest index among equals, in every lane of the row.  Four DPP
// moves (xor 1 and xor 2 inside quads, then the 8-lane and 16-lane mirrors)
// instead of LDS-routed shuffles.
template <int CTRL>
__device__ __forceinline__ void dpp_max_step(float& v, int& id) {
  const float ov = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
  const int oi = __builtin_amdgcn_mov_dpp(id, CTRL, 0xF, 0xF, false);
  const bool take = (ov > v) | ((ov == v) & (oi < id));
  v = take ? ov : v;
  id = take ? oi : id;
}
__device__ __forceinline__ void row16_max_lowid(float& v, int& id) {
  dpp_max_step<0xB1>(v, id);    // quad_perm [1, 0, 3, 2]
  dpp_max_step<0x4E>(v, id);    // quad_perm [2, 3, 0, 1]
  dpp_max_step<0x141>(v, id);   // row_half_mirror
  dpp_max_step<0x140>(v, id);   // row_mirror
}

// RoPE: the angle pos * theta^(-2j/dh) of pair j, reduced to [-pi, pi] in
// double, then evaluated in float.
// Frequency of pair j: theta^(-2 j / dh), in double.
__device__ __forceinline__ double rope_inv_freq(int j, int dh, float theta) {
  return exp(-2.0 * static_cast<double>(j) / dh * log(static_cast<double>(theta)));
}

// cos / sin of the angle pos * inv, reduced to [-pi, pi] in double first.
__device__ __forceinline__ void rope_cos_sin_at(int pos, double inv, float* c, float* s) {
  double ang = static_cast<double>(pos) * inv;
  const double two_pi = 6.283185307179586476925286766559;
  ang -= two_pi * rint(ang / two_pi);
  sincosf(static_cast<float>(ang), s, c);
}

__device__ __forceinline__ void rope_cos_sin(int pos, int j, int dh, float theta, float* c,
                                             float* s) {
  rope_cos_sin_at(pos, rope_inv_freq(j, dh, theta), c, s);
}

// Step gate of the adaptive block loop: a kernel handed a non-null n_done
// returns at once when n_done[0] >= n, i.e. every row of the batch has
// stopped (the steps the host queued ahead of its done check then cost only
// their launches).  The count is read once per workgroup, through lane 0.
__device__ __forceinline__ bool step_gate_closed(const int32_t* n_done, int n) {
  return n_done != nullptr && __builtin_amdgcn_readfirstlane(*n_done) >= n;
}

// s_waitcnt immediates: vector-memory count <= n (bits 3:0 and 15:14), export
// and LDS/scalar counts left at their maxima (no wait on them)
constexpr int waitcnt_vm(int n) { return (n & 0xf) | (0x7 << 4) | (0xf << 8) | (((n >> 4) & 3) << 14); }

// Logical workgroup index for a grid of a multiple of 8 workgroups:
// hardware deals linear workgroup ids round-robin over the 8 XCDs, so this
// gives each XCD one contiguous range of logical indices (work items that
// share operands, placed at adjacent logical indices, share one L2).
__device__ __forceinline__ int xcd_logical_tile(int linear, int total) {
  const int per = (total + 7) / 8;
  return (linear % 8) * per + linear / 8;
}

}  // namespace dg
