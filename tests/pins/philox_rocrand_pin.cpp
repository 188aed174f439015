// Independent Philox4x32-10 reference for the oracle's tests: prints
// rocRAND's host-side Philox4x32-10 output for counters and keys read from
// stdin ("c0 c1 c2 c3 k0 k1" in hex, one set per line).  rocRAND maps
// (seed, subsequence, offset) to key = seed, counter.zw = subsequence,
// counter.xy = offset / 4, so any counter with c1 < 2^30 is reachable.
#include <cstdio>
#include <cstdint>
#include <rocrand/rocrand_philox4x32_10.h>

int main() {
  unsigned c0, c1, c2, c3, k0, k1;
  while (std::scanf("%x %x %x %x %x %x", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    unsigned long long seed = ((unsigned long long)k1 << 32) | k0;
    unsigned long long subseq = ((unsigned long long)c3 << 32) | c2;
    unsigned long long offset = 4ull * (((unsigned long long)c1 << 32) | c0);
    rocrand_state_philox4x32_10 st;
    rocrand_init(seed, subseq, offset, &st);
    uint4 r = rocrand4(&st);
    std::printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
