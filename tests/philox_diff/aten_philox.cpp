// Differential check helper: evaluates Philox4x32-10 through PyTorch's open-source
// PhiloxRNGEngine header (compiled and run here, nothing copied). Reads lines
// "c0 c1 c2 c3 k0 k1" (hex) on stdin, prints the four output words (hex).
// The engine is constructed as (seed = k1:k0, subsequence = c3:c2, offset = c1:c0), which
// places exactly that counter and key in its state; operator() then returns words 0..3.
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>
#include <cstdint>

int main() {
  unsigned c0, c1, c2, c3, k0, k1;
  while (std::scanf("%x %x %x %x %x %x", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    uint64_t seed = ((uint64_t)k1 << 32) | k0;
    uint64_t subseq = ((uint64_t)c3 << 32) | c2;
    uint64_t offset = ((uint64_t)c1 << 32) | c0;
    at::Philox4_32 eng(seed, subseq, offset);
    uint32_t w0 = eng(), w1 = eng(), w2 = eng(), w3 = eng();
    std::printf("%08x %08x %08x %08x\n", w0, w1, w2, w3);
  }
  return 0;
}
