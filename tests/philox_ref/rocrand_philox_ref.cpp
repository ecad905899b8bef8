// Independent Philox4x32-10 outputs for pinning the oracle: the host side of
// rocRAND's header-only philox4x32_10 engine (a third-party implementation of
// Salmon et al., SC'11).  Prints the first N 32-bit outputs of the stream with
// the given seed and subsequence, one per line.  Built and run by the CPU test
// suite only.
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>
#include <cstdlib>

int main(int argc, char** argv) {
  if (argc != 4) {
    std::fprintf(stderr, "usage: %s seed subsequence count\n", argv[0]);
    return 2;
  }
  const unsigned long long seed = std::strtoull(argv[1], nullptr, 0);
  const unsigned long long subseq = std::strtoull(argv[2], nullptr, 0);
  const unsigned long long n = std::strtoull(argv[3], nullptr, 0);
  rocrand_device::philox4x32_10_engine eng(seed, subseq, 0);
  for (unsigned long long i = 0; i < n; ++i) std::printf("%u\n", eng.next());
  return 0;
}
