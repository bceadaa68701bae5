// Witness: PyTorch's header-only Philox4x32-10 engine, run on the host.
// Reads lines "seed subsequence offset" (decimal uint64) from stdin and prints
// the four 32-bit words of the first block of each stream in hex.
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>
#include <cinttypes>

int main() {
  unsigned long long seed, sub, off;
  while (std::scanf("%llu %llu %llu", &seed, &sub, &off) == 3) {
    at::philox_engine e(seed, sub, off);
    uint32_t w0 = e(), w1 = e(), w2 = e(), w3 = e();
    std::printf("%08x %08x %08x %08x\n", w0, w1, w2, w3);
  }
  return 0;
}
