// Independent Philox4x32-10 pin: rocRAND's engine (public header, host path).
// Reads lines "k0 k1 c0 c1 c2 c3" (hex) and prints the four output words.
// Counter mapping: rocRAND's engine(seed, subsequence, offset) starts from
// counter (offset/4 as words 0-1, subsequence as words 2-3), so
// seed = k1:k0, subsequence = c3:c2, and an offset of 4 * (c1:c0) numbers,
// applied as 4*c0 and then four skips of c1 << 32 (4 * (c1:c0) can overflow).
#include <cstdio>
#include <rocrand/rocrand_philox4x32_10.h>

int main() {
  unsigned k0, k1, c0, c1, c2, c3;
  while (std::scanf("%x %x %x %x %x %x", &k0, &k1, &c0, &c1, &c2, &c3) == 6) {
    unsigned long long seed = ((unsigned long long)k1 << 32) | k0;
    unsigned long long sub = ((unsigned long long)c3 << 32) | c2;
    rocrand_device::philox4x32_10_engine eng(seed, sub, 4ull * c0);
    for (int t = 0; t < 4; ++t) eng.discard((unsigned long long)c1 << 32);
    uint4 o = eng.next4();
    std::printf("%08x %08x %08x %08x\n", o.x, o.y, o.z, o.w);
  }
  return 0;
}
