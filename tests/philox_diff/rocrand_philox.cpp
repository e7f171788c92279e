// Differential check helper: evaluates Philox4x32-10 through rocRAND's open-source
// philox4x32_10_engine header (compiled and run on the host, nothing copied). The engine's
// protected ten_rounds(counter, key) is reached through a derived class. Same stdin/stdout
// format as aten_philox.cpp.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

struct probe : rocrand_device::philox4x32_10_engine {
  uint4 run(uint4 c, uint2 k) { return this->ten_rounds(c, k); }
};

int main() {
  unsigned c0, c1, c2, c3, k0, k1;
  probe p;
  while (std::scanf("%x %x %x %x %x %x", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    uint4 c; c.x = c0; c.y = c1; c.z = c2; c.w = c3;
    uint2 k; k.x = k0; k.y = k1;
    uint4 o = p.run(c, k);
    std::printf("%08x %08x %08x %08x\n", o.x, o.y, o.z, o.w);
  }
  return 0;
}
