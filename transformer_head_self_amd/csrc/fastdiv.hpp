// Division by a divisor fixed at launch time, as a multiply-high, an add and
// a shift (Granlund and Montgomery, "Division by invariant integers using
// multiplication", PLDI 1994, the round-up method for unsigned operands):
// with l = ceil(log2 d) and magic = floor(2^32 (2^l - d) / d) + 1,
//   n / d == (umulhi(n, magic) + n) >> l    for 0 <= n < 2^31, 1 <= d < 2^31.
// (n < 2^31 keeps the sum of the two terms below 2^32.)
// Plain C++: usable from host code, from kernels and from a CPU test.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define MHA_HOST_DEVICE __host__ __device__
#else
#define MHA_HOST_DEVICE
#endif

namespace mha {

struct FastDiv {
  uint32_t magic;
  uint32_t shift;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  const uint64_t magic = ((1ull << 32) * ((1ull << l) - d)) / d + 1;
  return FastDiv{(uint32_t)magic, l};
}

MHA_HOST_DEVICE inline uint32_t fastdiv(uint32_t n, FastDiv f) {
  const uint32_t hi = (uint32_t)(((uint64_t)n * f.magic) >> 32);
  return (hi + n) >> f.shift;
}

}  // namespace mha
