// Reference Philox4x32-10 outputs from rocRAND's header-only engine, run on the
// host.  Used by the CPU tests to pin the oracle's own Philox implementation to
// an independent one.  rocRAND's engine is addressed by (seed, subsequence,
// offset): the key is the seed, counter words 0-1 hold offset/4 and words 2-3
// hold the subsequence, so counter (c0, c1, c2, c3) is reached with
// subsequence = c2 | c3 << 32 and an offset of 4 * (c0 | c1 << 32), applied as
// 4 * c0 at construction plus four discards of c1 << 32 (each advancing the
// counter by c1 << 30) so that no 64-bit offset overflows.
//
// stdin: lines "seed c0 c1 c2 c3"; stdout: lines "x0 x1 x2 x3" (decimal).
#include <cstdio>
#include <rocrand/rocrand_philox4x32_10.h>

int main() {
  unsigned long long seed;
  unsigned int c[4];
  while (std::scanf("%llu %u %u %u %u", &seed, &c[0], &c[1], &c[2], &c[3]) == 5) {
    unsigned long long sub = (unsigned long long)c[2] | ((unsigned long long)c[3] << 32);
    rocrand_device::philox4x32_10_engine eng(seed, sub, 4ull * c[0]);
    for (int r = 0; r < 4; ++r) eng.discard((unsigned long long)c[1] << 32);
    unsigned int x0 = eng(), x1 = eng(), x2 = eng(), x3 = eng();
    std::printf("%u %u %u %u\n", x0, x1, x2, x3);
  }
  return 0;
}
