// Witness: rocRAND's Philox4x32-10 host implementation.  Same I/O as
// philox_torch.cpp; rocRAND counts its offset in 32-bit draws, so a stream
// offset of `off` blocks is requested as 4 * off draws.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
#include <cinttypes>

int main() {
  unsigned long long seed, sub, off;
  while (std::scanf("%llu %llu %llu", &seed, &sub, &off) == 3) {
    rocrand_state_philox4x32_10 s;
    rocrand_init(seed, sub, off * 4ull, &s);
    uint32_t w0 = rocrand(&s), w1 = rocrand(&s), w2 = rocrand(&s), w3 = rocrand(&s);
    std::printf("%08x %08x %08x %08x\n", w0, w1, w2, w3);
  }
  return 0;
}
