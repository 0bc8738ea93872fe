// Host-only helper for the oracle's Philox pin: runs ROCm's rocRAND
// Philox4x32-10 block function (an independent library implementation of
// Salmon et al., SC'11) on (counter, key) tuples read from stdin, one tuple
// of six hex words per line, and prints the four output words.
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>

struct PhiloxBlock : rocrand_device::philox4x32_10_engine {
  uint4 run(uint4 counter, uint2 key) { return ten_rounds(counter, key); }
};

int main() {
  PhiloxBlock p;
  unsigned c0, c1, c2, c3, k0, k1;
  while (std::scanf("%x %x %x %x %x %x", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    uint4 r = p.run(uint4{c0, c1, c2, c3}, uint2{k0, k1});
    std::printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
