// Test helper: prints rocRAND's Philox4x32-10 output for (key, counter) pairs read from stdin,
// one "key ctr0 ctr1 ctr2 ctr3" line per query (decimal). Host code only: rocRAND's engine is
// host-callable. The engine is positioned on the requested counter through its public
// seed / subsequence / offset interface: subsequence fills counter words 2-3, offset/4 words 0-1.
#include <cstdio>
#include <rocrand/rocrand_philox4x32_10.h>

int main() {
  unsigned long long key;
  unsigned int c0, c1, c2, c3;
  while (std::scanf("%llu %u %u %u %u", &key, &c0, &c1, &c2, &c3) == 5) {
    const unsigned long long subsequence = c2 | (static_cast<unsigned long long>(c3) << 32);
    const unsigned long long offset = 4ull * (c0 | (static_cast<unsigned long long>(c1) << 32));
    rocrand_device::philox4x32_10_engine eng(key, subsequence, offset);
    const uint4 r = eng.next4();
    std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
