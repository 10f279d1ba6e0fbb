// Test helper: prints Philox4x32-10 outputs from rocRAND's header-only
// engine, as an independent check of the oracle's Philox.  Reads lines
// "key_lo key_hi c0 c1 c2 c3" (decimal) on stdin and prints the four output
// words in hex.  rocRAND's engine(seed, subsequence, offset) starts from
// counter (offset/4 as 64 bits, subsequence as 64 bits).
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

int main() {
  unsigned long long klo, khi, c0, c1, c2, c3;
  while (std::scanf("%llu %llu %llu %llu %llu %llu", &klo, &khi, &c0, &c1, &c2, &c3) == 6) {
    unsigned long long seed = klo | (khi << 32);
    unsigned long long sub = c2 | (c3 << 32);
    unsigned long long ctr01 = c0 | (c1 << 32);
    rocrand_device::philox4x32_10_engine e(seed, sub, 0);
    e.discard(4ull * ctr01);   // counter words 0,1 += ctr01 (exact below 2^62)
    unsigned a = e.next(), b = e.next(), c = e.next(), d = e.next();
    std::printf("%08x %08x %08x %08x\n", a, b, c, d);
  }
  return 0;
}
