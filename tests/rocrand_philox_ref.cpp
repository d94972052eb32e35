// Known-answer source for the oracle's Philox4x32-10: rocRAND's engine,
// compiled for the host. Reads lines "c0 c1 c2 c3 k0 k1" (hex words) and
// prints the four output words of one Philox4x32-10 call for that counter
// and key. rocRAND seeds key = (seed lo, seed hi), puts the subsequence in
// counter words 2..3 and offset/4 in counter words 0..1.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

int main() {
  unsigned c0, c1, c2, c3, k0, k1;
  while (std::scanf("%x %x %x %x %x %x", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    unsigned long long seed = (unsigned long long)k1 << 32 | k0;
    unsigned long long subseq = (unsigned long long)c3 << 32 | c2;
    unsigned long long offset = ((unsigned long long)c1 << 32 | c0) * 4ull;
    rocrand_device::philox4x32_10_engine e(seed, subseq, offset);
    uint4 r = e.next4();
    std::printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
