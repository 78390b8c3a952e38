// Prints words of rocRAND's host-side Philox4x32-10 engine, one hex word per line.
// Used only by the oracle's tests as an independent implementation of the
// generator: rocRAND keys the engine with the 64-bit seed and starts the
// 128-bit counter at (offset / 4, subsequence << 64).
// usage: rocrand_philox_kat SEED SUBSEQUENCE OFFSET COUNT
#include <rocrand/rocrand_kernel.h>
#include <cstdio>
#include <cstdlib>

int main(int argc, char** argv) {
  if (argc != 5) return 2;
  const unsigned long long seed = strtoull(argv[1], nullptr, 0);
  const unsigned long long subseq = strtoull(argv[2], nullptr, 0);
  const unsigned long long offset = strtoull(argv[3], nullptr, 0);
  const long n = strtol(argv[4], nullptr, 0);
  rocrand_state_philox4x32_10 st;
  rocrand_init(seed, subseq, offset, &st);
  for (long i = 0; i < n; ++i) printf("%08x\n", rocrand(&st));
  return 0;
}
