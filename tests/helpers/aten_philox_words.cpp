// Test helper: prints the four Philox4x32-10 words that PyTorch's own
// header-only engine (ATen/core/PhiloxRNGEngine.h) produces for each
// (counter, key) read from stdin, one "c0 c1 c2 c3 k0 k1" line each.
// The engine keys on the 64-bit seed and counts with
// counter = (offset_lo, offset_hi, subsequence_lo, subsequence_hi), so an
// arbitrary counter is reached by choosing offset and subsequence.
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdint>
#include <cstdio>

int main() {
  unsigned long long c0, c1, c2, c3, k0, k1;
  while (std::scanf("%llu %llu %llu %llu %llu %llu", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    uint64_t seed = (uint64_t)k0 | ((uint64_t)k1 << 32);
    uint64_t subsequence = (uint64_t)c2 | ((uint64_t)c3 << 32);
    uint64_t offset = (uint64_t)c0 | ((uint64_t)c1 << 32);
    at::Philox4_32 engine(seed, subsequence, offset);
    uint32_t w0 = engine(), w1 = engine(), w2 = engine(), w3 = engine();
    std::printf("%u %u %u %u\n", w0, w1, w2, w3);
  }
  return 0;
}
