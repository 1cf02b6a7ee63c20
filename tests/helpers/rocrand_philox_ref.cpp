// Host-side reference for the oracle's Philox4x32-10: rocRAND's engine, used as a
// library routine. Reads lines "seed b h i" and prints the four 32-bit outputs of
// the counter (i, h, b, 0) under the key (seed low word, seed high word).
// Test infrastructure only; compiled by the CPU tests with the host compiler.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

int main() {
  unsigned long long seed, b, h, i;
  while (std::scanf("%llu %llu %llu %llu", &seed, &b, &h, &i) == 4) {
    // subsequence b fills counter words 2..3; offset 4*(h<<32 | i) fills words 0..1.
    rocrand_device::philox4x32_10_engine e(seed, b, 4ull * ((h << 32) | i));
    uint4 r = e.next4();
    std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
