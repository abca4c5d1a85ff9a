// Host-side reference for the Philox-4x32-10 pin: runs rocRAND's own
// Philox-4x32-10 round function (the engine in rocrand_philox4x32_10.h,
// compiled here for the CPU) on (counter, key) tuples read from stdin, one
// "c0 c1 c2 c3 k0 k1" line each, and prints the four output words.
// Test infrastructure only; built by tests/test_oracle_dropout.py.
#include <cstdio>

#include <rocrand/rocrand_philox4x32_10.h>

namespace {
struct Rounds : rocrand_device::philox4x32_10_engine {
  uint4 run(uint4 counter, uint2 key) { return ten_rounds(counter, key); }
};
}  // namespace

int main() {
  Rounds engine;
  unsigned c0, c1, c2, c3, k0, k1;
  while (std::scanf("%u %u %u %u %u %u", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    const uint4 r = engine.run(uint4{c0, c1, c2, c3}, uint2{k0, k1});
    std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
