// Philox4x32-10 blocks from rocRAND's engine (rocrand_philox4x32_10.h, its
// host-callable device API), for the oracle's generator pin.  Reads lines
// "seed subsequence n" and prints the four 32-bit words of the block at
// counter (n mod 2^32, n div 2^32, subsequence mod 2^32, subsequence div 2^32)
// under key (seed mod 2^32, seed div 2^32): the engine seeded with seed, moved
// to that subsequence and to offset 4 n returns that block's words in order.
#include <cstdio>

#include <rocrand/rocrand_philox4x32_10.h>

int main() {
  unsigned long long seed, sub, n;
  while (std::scanf("%llu %llu %llu", &seed, &sub, &n) == 3) {
    rocrand_device::philox4x32_10_engine e(seed, sub, 4 * n);
    const unsigned a = e(), b = e(), c = e(), d = e();
    std::printf("%u %u %u %u\n", a, b, c, d);
  }
  return 0;
}
