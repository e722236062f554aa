// Prints rocRAND's Philox4x32-10 output block for (seed, b, t, j) read from stdin,
// with counter (j, t, b, 0) and key (seed lo, seed hi).  Host-only helper that pins
// the CPU oracle's Philox to an independent, published implementation.
#include <rocrand/rocrand_kernel.h>
#include <cstdio>

int main() {
  unsigned long long seed, b, t, j;
  while (std::scanf("%llu %llu %llu %llu", &seed, &b, &t, &j) == 4) {
    rocrand_state_philox4x32_10 st;
    rocrand_init(seed, b, 4ull * (j + (t << 32)), &st);
    unsigned int w0 = rocrand(&st), w1 = rocrand(&st), w2 = rocrand(&st), w3 = rocrand(&st);
    std::printf("%u %u %u %u\n", w0, w1, w2, w3);
  }
  return 0;
}
