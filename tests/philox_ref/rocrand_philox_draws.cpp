// Philox4x32-10 words from rocRAND's open-source, host-callable engine, an
// implementation of the generator of Salmon et al. (SC'11) that shares nothing
// with the oracle.  It pins the oracle's generator and its counter layout:
// for each input line "seed subsequence offset" the program prints the first
// word the engine yields after seeding with (seed, subsequence, offset).  The
// engine keys the rounds with the seed, puts the subsequence in counter words
// 2-3 and offset / 4 in counter words 0-1, and yields word offset % 4 first --
// the oracle's (seed, SR offset, element index) layout.  Host code only.
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>

int main() {
  unsigned long long seed, subsequence, offset;
  while (std::scanf("%llu %llu %llu", &seed, &subsequence, &offset) == 3) {
    rocrand_device::philox4x32_10_engine engine(seed, subsequence, offset);
    std::printf("%u\n", engine.next());
  }
  return 0;
}
