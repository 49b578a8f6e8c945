// Test-only helper: prints Philox4x32-10 outputs from the rocRAND header
// implementation, used as an independent known-answer source for the
// oracle's own Philox.  Never linked into the oracle or the HIP library.
// Input lines on stdin: key counter0 counter1 counter2 counter3 (decimal).
// Output lines: the four 32-bit words of the block function.
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdint>
#include <cstdio>

int main() {
  unsigned long long key, c0, c1, c2, c3;
  while (std::scanf("%llu %llu %llu %llu %llu", &key, &c0, &c1, &c2, &c3) == 5) {
    // engine(seed, subsequence, offset): key = seed, counter.zw = subsequence,
    // counter.xy = offset / 4; draws come out as words x, y, z, w.
    unsigned long long g = c0 | (c1 << 32);
    unsigned long long sub = c2 | (c3 << 32);
    rocrand_device::philox4x32_10_engine eng(key, sub, 4ull * g);
    unsigned w0 = eng(), w1 = eng(), w2 = eng(), w3 = eng();
    std::printf("%u %u %u %u\n", w0, w1, w2, w3);
  }
  return 0;
}
