// Independent Philox4x32-10 for pinning the oracle's generator: rocRAND's
// host-callable engine.  Reads "c0 c1 c2 c3 seed" lines (decimal) on stdin and
// prints the four output words of ten rounds on that counter under the key
// (seed mod 2^32, seed >> 32).  rocRAND sets counter (x, y) from offset / 4
// and (z, w) from the subsequence, so the requested counter maps to
// subsequence = c2 | c3 << 32 and offset = 4 * (c0 | c1 << 32) (c1 < 2^30).
#include <cstdio>
#include <rocrand/rocrand_philox4x32_10.h>

int main() {
  unsigned long long c0, c1, c2, c3, seed;
  while (std::scanf("%llu %llu %llu %llu %llu", &c0, &c1, &c2, &c3, &seed) == 5) {
    rocrand_device::philox4x32_10_engine eng(seed, c2 | (c3 << 32), 4ull * (c0 | (c1 << 32)));
    uint4 r = eng.next4();
    std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
