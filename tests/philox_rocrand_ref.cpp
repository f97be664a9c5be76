// Reference outputs of Philox4x32-10 from rocRAND's header implementation,
// run on the host: reads lines "seed c0 c1 c2 c3" (decimal) and prints the four
// output words of the generator at that 128-bit counter under key seed.
// rocRAND's state maps the counter as: (c0, c1) = offset / 4, (c2, c3) =
// subsequence, so rocrand_init(seed, c2 + 2^32 c3, 4 (c0 + 2^32 c1)) followed by
// one rocrand4() returns the block at that counter (the offset is 64-bit, so
// c1 < 2^30).
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>

int main() {
  unsigned long long seed, c0, c1, c2, c3;
  while (std::scanf("%llu %llu %llu %llu %llu", &seed, &c0, &c1, &c2, &c3) == 5) {
    rocrand_state_philox4x32_10 st;
    rocrand_init(seed, c2 | (c3 << 32), 4ull * (c0 | (c1 << 32)), &st);
    const uint4 w = rocrand4(&st);
    std::printf("%u %u %u %u\n", w.x, w.y, w.z, w.w);
  }
  return 0;
}
