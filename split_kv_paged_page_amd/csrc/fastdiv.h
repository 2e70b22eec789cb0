// Division by a launch-time constant as a multiply-high, add and shift
// (the round-up method of Granlund and Montgomery, "Division by Invariant
// Integers using Multiplication", PLDI 1994): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, n / d = (mulhi(n, m) + n) >> l for every
// n < 2^31.  The host computes (m, l) once per launch; the kernels divide
// workgroup ids, context lengths and row indices without the long
// reciprocal sequence a runtime divisor costs on the vector ALUs.
#pragma once

#include <stdint.h>

namespace splitkv {

struct FastDiv {
  uint32_t mul;
  uint32_t shift;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((uint64_t(1) << l) < d) ++l;
  const uint64_t m = (((uint64_t(1) << l) - d) << 32) / d + 1;
  return FastDiv{uint32_t(m), l};
}

// n < 2^31.
__host__ __device__ inline uint32_t fdiv(uint32_t n, FastDiv f) {
  const uint32_t t = uint32_t((uint64_t(n) * f.mul) >> 32);
  return (t + n) >> f.shift;
}

}  // namespace splitkv
