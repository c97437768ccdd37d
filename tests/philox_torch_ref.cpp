// Host-only helper for the oracle's Philox pin: runs PyTorch's open-source
// philox_engine (ATen/core/PhiloxRNGEngine.h) as a black box.  Reads lines
// "c0 c1 c2 c3 k0 k1" (decimal uint32) from stdin, prints the four outputs.
// The engine is seeded with key = seed (lo, hi); its counter starts at
// (0, 0, subsequence_lo, subsequence_hi) and advances by `offset` 128-bit
// steps, so seed=(k1<<32|k0), subsequence=(c3<<32|c2), offset=(c1<<32|c0)
// places the counter at exactly (c0, c1, c2, c3).
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>
#include <cstdint>
int main() {
  unsigned long long c0, c1, c2, c3, k0, k1;
  while (std::scanf("%llu %llu %llu %llu %llu %llu", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    uint64_t seed = (k1 << 32) | k0;
    uint64_t subseq = (c3 << 32) | c2;
    uint64_t offset = (c1 << 32) | c0;
    at::philox_engine eng(seed, subseq, offset);
    uint32_t a = eng(), b = eng(), c = eng(), d = eng();
    std::printf("%u %u %u %u\n", a, b, c, d);
  }
  return 0;
}
