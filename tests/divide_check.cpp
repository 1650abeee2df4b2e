// divide_check.cpp -- host check of the exact multiply-high division used by the
// flat kernels (modulation_bf16_row_amd/csrc/dit_divide.hpp): the library's own
// reciprocal() with a host stand-in for the device's 64-bit multiply-high.
// Exhaustive over all 2^32 numerators for the divisors named on the command
// line after "--all", edge and pseudo-random numerators for the others.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dit_divide.hpp"

static uint32_t div_host(uint32_t n, uint64_t m) {
  return m ? (uint32_t)(((unsigned __int128)n * m) >> 64) : n;
}

static long check(uint64_t d, bool all) {
  const uint64_t m = dit::reciprocal(d);
  long bad = 0;
  if (all) {
    for (uint64_t n = 0; n <= 0xFFFFFFFFull; ++n)
      if (div_host((uint32_t)n, m) != (uint32_t)n / d) ++bad;
    return bad;
  }
  const uint32_t edges[] = {0u, 1u, 2u, (uint32_t)(d - 1), (uint32_t)d, (uint32_t)(d + 1),
                            (uint32_t)(2 * d - 1), 0x7FFFFFFFu, 0x80000000u, 0xFFFFFFFEu,
                            0xFFFFFFFFu};
  for (uint32_t n : edges)
    if (div_host(n, m) != n / d) ++bad;
  uint64_t x = 0x9E3779B97F4A7C15ull ^ d;
  for (int i = 0; i < 4000000; ++i) {
    x ^= x << 13; x ^= x >> 7; x ^= x << 17;
    const uint32_t n = (uint32_t)x;
    if (div_host(n, m) != n / d) ++bad;
    const uint32_t q = n / d;                 // multiples and their neighbours
    const uint32_t k = (uint32_t)(q * d);
    if (div_host(k, m) != k / d) ++bad;
    if (k && div_host(k - 1, m) != (k - 1) / d) ++bad;
  }
  return bad;
}

int main(int argc, char **argv) {
  long bad = 0;
  bool all = false;
  for (int i = 1; i < argc; ++i) {
    if (!strcmp(argv[i], "--all")) { all = true; continue; }
    const uint64_t d = strtoull(argv[i], nullptr, 10);
    const long b = check(d, all);
    if (b) printf("divisor %llu: %ld wrong quotients\n", (unsigned long long)d, b);
    bad += b;
  }
  printf("bad %ld\n", bad);
  return bad != 0;
}
