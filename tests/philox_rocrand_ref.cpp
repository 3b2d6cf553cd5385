// Host-side comparator for the oracle's Philox4x32: runs rocRAND's own
// header-only philox4x32_10 engine (ten rounds) on counter/key pairs read from
// stdin ("c0 c1 c2 c3 k0 k1" per line, decimal) and prints the four output
// words.  Used only by tests/test_oracle_philox.py.
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>

namespace {
struct Engine : rocrand_device::philox4x32_10_engine {
  Engine() : rocrand_device::philox4x32_10_engine(0, 0, 0) {}
  uint4 block(uint4 c, uint2 k) { return ten_rounds(c, k); }
};
}  // namespace

int main() {
  Engine e;
  unsigned c0, c1, c2, c3, k0, k1;
  while (std::scanf("%u %u %u %u %u %u", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    uint4 o = e.block(uint4{c0, c1, c2, c3}, uint2{k0, k1});
    std::printf("%u %u %u %u\n", o.x, o.y, o.z, o.w);
  }
  return 0;
}
