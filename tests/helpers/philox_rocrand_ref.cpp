// Prints the first N Philox4x32-10 blocks of rocRAND's engine (counters 0..N-1,
// key = seed) from its public header, run on the host.  Used only by the CPU
// test that pins the oracle's Philox against an independent implementation.
#include <rocrand/rocrand_kernel.h>
#include <cstdio>
#include <cstdlib>

int main(int argc, char** argv) {
  if (argc < 3) return 2;
  unsigned long long seed = strtoull(argv[1], nullptr, 0);
  int n = atoi(argv[2]);
  rocrand_state_philox4x32_10 st;
  rocrand_init(seed, 0, 0, &st);
  for (int i = 0; i < n; ++i) {
    uint4 v = rocrand4(&st);
    printf("%u %u %u %u\n", v.x, v.y, v.z, v.w);
  }
  return 0;
}
