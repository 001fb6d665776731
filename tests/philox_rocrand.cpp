// Host-only helper for the oracle's generator pin: prints the four words of
// rocRAND's Philox4x32-10 (documented interface: rocrand_init(seed,
// subsequence, offset) then rocrand4) for the blocks named on stdin, one
// "seed subsequence block" triple per line.  Runs no device code.
#include <rocrand/rocrand_kernel.h>

#include <cstdio>

int main() {
  unsigned long long seed, sub, block;
  while (std::scanf("%llu %llu %llu", &seed, &sub, &block) == 3) {
    rocrand_state_philox4x32_10 s;
    rocrand_init(seed, sub, 4ull * block, &s);
    const uint4 v = rocrand4(&s);
    std::printf("%u %u %u %u\n", v.x, v.y, v.z, v.w);
  }
  return 0;
}
