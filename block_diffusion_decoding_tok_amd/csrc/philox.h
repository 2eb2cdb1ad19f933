// Philox4x32-10 on the device, written from its published definition
// (Salmon, Moraes, Dror, Shaw: "Parallel Random Numbers: As Easy as 1, 2, 3",
// SC'11).  One round: (c0, c1, c2, c3) -> (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2),
// hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)); ten rounds with the key advanced by the
// Weyl increments between rounds.  Key = (seed lo, seed hi).
//
// Counter layout used by the sampler: (word, absolute position, step,
// (stream << 24) | row) with streams 0 = Gumbel, 1 = re-noise id, 2 = initial
// canvas id.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;

enum : uint32_t { kStreamGumbel = 0, kStreamRenoise = 1, kStreamCanvas = 2 };

struct Philox4 {
  uint32_t x, y, z, w;
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = static_cast<uint64_t>(kPhiloxM0) * c0;
    const uint64_t p1 = static_cast<uint64_t>(kPhiloxM1) * c2;
    // three-input xors in one v_bitop3_b32 each (truth table 0x96)
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32(static_cast<uint32_t>(p1 >> 32), c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32(static_cast<uint32_t>(p0 >> 32), c3, k1, 0x96);
    c1 = static_cast<uint32_t>(p1);
    c3 = static_cast<uint32_t>(p0);
    c0 = n0;
    c2 = n2;
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
  return Philox4{c0, c1, c2, c3};
}

// Uniform integer in [0, n): floor(w * n / 2^32).
__device__ __forceinline__ uint32_t uniform_id(uint32_t w, uint32_t n) {
  return static_cast<uint32_t>((static_cast<uint64_t>(w) * n) >> 32);
}

// Standard Gumbel draw g = -ln(-ln u), u = ((w >> 8) + 1/2) 2^-24, in float.
// u carries up to 25 significant bits, so float holds u exactly only below
// 1/2.  Above, t = 1 - u is exact and ln u = ln(fl(u)) + ((1 - fl(u)) - t)
// to first order (the correction is at most 2^-25 relative to fl(u)), which
// keeps -ln u accurate in relative terms all the way to u -> 1.
__device__ __forceinline__ float gumbel_from_word(uint32_t w) {
  const uint32_t k = w >> 8;
  const float kf = static_cast<float>(k);                       // exact (< 2^24)
  const float u = __builtin_fmaf(kf, 0x1.0p-24f, 0x1.0p-25f);   // fl(u)
  const float tf = static_cast<float>(0xFFFFFFu - k);           // exact
  const float t = __builtin_fmaf(tf, 0x1.0p-24f, 0x1.0p-25f);   // exact when k >= 2^23
  const float corr = (k >= 0x800000u) ? ((1.0f - u) - t) : 0.0f;
  const float ln2 = 0.693147180559945309f;
  const float neg_ln_u = -(__builtin_amdgcn_logf(u) * ln2 + corr);
  return -__builtin_amdgcn_logf(neg_ln_u) * ln2;
}

}  // namespace dg
