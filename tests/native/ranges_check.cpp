// Host-side check of the decode kernel's range arithmetic (attn::Ranges):
// for many block totals T and range counts P, lo(i) equals floor(i T / P)
// and owner(x) is the largest i with lo(i) <= x, against plain integer
// arithmetic.  Compiled for the host only; prints "ok" or the first
// mismatch and exits nonzero.
#include <cstdio>
#include <cstdlib>

#include "decode.hpp"

static long long lo_ref(long long T, int P, int i) {
  return (long long)((__int128)T * i / P);
}

static int check(long long T, int P) {
  const attn::Ranges rg(T, P);
  for (int i = 0; i <= P; ++i)
    if (rg.lo(i) != lo_ref(T, P, i)) {
      std::printf("lo mismatch T=%lld P=%d i=%d: %lld vs %lld\n", T, P, i,
                  rg.lo(i), lo_ref(T, P, i));
      return 1;
    }
  // owner at every range start and end, and a spread of blocks between
  for (int i = 0; i < P; ++i) {
    const long long a = lo_ref(T, P, i), b = lo_ref(T, P, i + 1);
    if (a == b) continue;                  // empty range holds no block
    const long long xs[4] = {a, b - 1, a + (b - a) / 2, a + (b - a) / 3};
    for (long long x : xs)
      if (rg.owner(x) != i) {
        std::printf("owner mismatch T=%lld P=%d x=%lld: %d vs %d\n", T, P, x,
                    rg.owner(x), i);
        return 1;
      }
  }
  return 0;
}

int main() {
  const int Ps[] = {1, 2, 3, 7, 16, 37, 255, 256, 512, 1000, 1024, 4096};
  long long Ts[64];
  int n = 0;
  for (long long t : {1LL, 2LL, 3LL, 5LL, 17LL, 255LL, 256LL, 257LL, 4559LL,
                      4592LL, 100003LL, 9999991LL, (1LL << 31) - 1,
                      (1LL << 31) + 7, (1LL << 35) + 12345,
                      (1LL << 40) - 1})
    Ts[n++] = t;
  srand(1);
  while (n < 64) Ts[n++] = 1 + ((long long)rand() << 16 ^ rand()) % (1LL << 39);
  for (int k = 0; k < n; ++k)
    for (int P : Ps)
      if (check(Ts[k], P)) return 1;
  std::printf("ok\n");
  return 0;
}
