// Division by a divisor fixed for a whole launch, with one high multiply, one add and one
// shift instead of the ~25-instruction integer division sequence the compiler emits for a
// runtime divisor (on MI355X each such sequence on a work item's critical path costs about
// 0.08 us of latency per wave).
//
// The method is Granlund & Montgomery, "Division by invariant integers using
// multiplication" (PLDI 1994), unsigned case: for a divisor 1 <= d <= 2^31 let l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, which fits 32 bits; then for 0 <= n < 2^31,
//   n / d = (mulhi(m, n) + n) >> l,
// where the sum stays below 2^32 because mulhi(m, n) < n. (d = 1 gives l = 0, m = 1.)
// Plain C++ (no HIP types), so the host build and a host test can use it as well.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define MOL_HD __host__ __device__
#else
#define MOL_HD
#endif

namespace mol {

struct FastDiv {
  uint32_t d;  // the divisor, 1 <= d <= 2^31
  uint32_t m;  // the multiplier
  uint32_t l;  // the shift, ceil(log2 d)
};

// Host: the constants for divisor d, 1 <= d <= 2^31 (0 is treated as 1, larger as 2^31;
// every divisor here is a size or a count of at most 2^31 - 1).
inline FastDiv make_fastdiv(uint32_t d) {
  if (d == 0) d = 1;
  if (d > 0x80000000u) d = 0x80000000u;
  uint32_t l = 0;
  while (l < 32 && (uint64_t(1) << l) < d) ++l;
  const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
  return FastDiv{d, (uint32_t)m, l};
}

MOL_HD inline uint32_t mulhi32(uint32_t a, uint32_t b) {
  return (uint32_t)(((uint64_t)a * b) >> 32);
}

// n / d and n % d for 0 <= n < 2^31
MOL_HD inline int fdiv(int n, FastDiv f) {
  const uint32_t u = (uint32_t)n;
  return (int)((mulhi32(f.m, u) + u) >> f.l);
}
MOL_HD inline int fmod(int n, FastDiv f) { return n - fdiv(n, f) * (int)f.d; }

}  // namespace mol
