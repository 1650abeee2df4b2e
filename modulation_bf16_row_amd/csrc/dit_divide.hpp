// dit_divide.hpp -- exact division of 32-bit indices by a divisor fixed for
// a launch, as one multiply-high (Granlund and Montgomery, "Division by
// invariant integers using multiplication", PLDI 1994).  For 2 <= d < 2^32
// and M = floor(2^64 / d) + 1, M d - 2^64 lies in (0, d], so for every
// n < 2^32 the error n (M d - 2^64) / 2^64 stays below 1 / d and
// floor(n M / 2^64) = floor(n / d).  M = 0 stands for d = 1.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

// Host: M for divisor d (1 <= d < 2^32).
inline uint64_t reciprocal(uint64_t d) {
  if (d < 2) return 0;
  const uint64_t q = ~0ull / d, rem = ~0ull % d;     // 2^64 - 1 = q d + rem
  return q + (rem == d - 1 ? 1 : 0) + 1;             // d | 2^64 exactly when rem == d - 1
}

// Device: floor(n / d) from M = reciprocal(d).
__device__ __forceinline__ uint32_t div_by(uint32_t n, uint64_t m) {
  return m ? (uint32_t)__umul64hi((uint64_t)n, m) : n;
}

}  // namespace dit
