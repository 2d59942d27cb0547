// Host program used by the oracle tests: evaluates the Philox4x32-10 block
// function through rocRAND's open-source engine (run as a library, not
// copied) so that the oracle's own Philox can be compared against it.
// stdin: lines "c0 c1 c2 c3 k0 k1" (hex); stdout: "r0 r1 r2 r3" (hex).
// The engine is positioned with seed = key, subsequence = (c2, c3) and
// offset = 4 * (c0, c1), so that its first four outputs are the block
// function at exactly that counter.
#include <hip/hip_runtime.h>
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

int main() {
  unsigned c0, c1, c2, c3, k0, k1;
  while (std::scanf("%x %x %x %x %x %x", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    unsigned long long seed = (unsigned long long)k0 | ((unsigned long long)k1 << 32);
    unsigned long long sub = (unsigned long long)c2 | ((unsigned long long)c3 << 32);
    unsigned long long off = 4ull * ((unsigned long long)c0 | ((unsigned long long)c1 << 32));
    rocrand_device::philox4x32_10_engine e(seed, sub, off);
    uint4 r = e.next4();
    std::printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
