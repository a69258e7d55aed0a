// Prints Philox4x32-10 words from rocRAND's own engine (an independent,
// library implementation of the SC'11 generator), for pinning the oracle.
// Usage: rocrand_philox_words SEED OFFSET_BLOCKS N_WORDS
// Output: N_WORDS decimal uint32 words, one per line, starting at block
// OFFSET_BLOCKS (counter = OFFSET_BLOCKS, 0, 0 in rocRAND's 128-bit counter).
#include <cstdio>
#include <cstdlib>
#include <rocrand/rocrand_philox4x32_10.h>

int main(int argc, char** argv) {
  if (argc != 4) return 2;
  unsigned long long seed = std::strtoull(argv[1], nullptr, 10);
  unsigned long long offset_blocks = std::strtoull(argv[2], nullptr, 10);
  long long n = std::atoll(argv[3]);
  rocrand_device::philox4x32_10_engine eng(seed, 0ull, 0ull);
  // skip whole blocks: advance by 4 words per block, in chunks that stay
  // inside rocRAND's 64-bit discard argument
  unsigned long long left = offset_blocks;
  const unsigned long long chunk = 1ull << 60;
  while (left) {
    unsigned long long step = left < chunk ? left : chunk;
    eng.discard(step * 4ull);
    left -= step;
  }
  for (long long i = 0; i < n; ++i) std::printf("%u\n", eng());
  return 0;
}
