// Pin for the oracle's Philox4x32-10: runs rocRAND's Philox4x32-10 engine (the
// installed header-only implementation, compiled for the host) for each
// (seed, q, offset) triple read from stdin and prints the four output words.
// rocRAND's engine takes key = seed, counter words (0,1) = q (via the offset
// argument, four numbers per counter step) and counter words (2,3) = the
// subsequence argument.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

int main() {
  unsigned long long seed, q, off;
  while (std::scanf("%llu %llu %llu", &seed, &q, &off) == 3) {
    rocrand_device::philox4x32_10_engine eng(seed, off, 4ULL * q);
    uint4 r = eng.next4();
    std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
