#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
#include <cstdlib>
int main(int argc, char** argv) {
  // args: seed stream idx...
  unsigned long long seed = strtoull(argv[1], 0, 0);
  unsigned long long stream = strtoull(argv[2], 0, 0);
  for (int i = 3; i < argc; ++i) {
    unsigned long long idx = strtoull(argv[i], 0, 0);
    unsigned long long off = 4ull * ((stream << 32) + (idx >> 2)) + (idx & 3);
    rocrand_device::philox4x32_10_engine e(seed, 0, off);
    printf("%u\n", e.next());
  }
}
