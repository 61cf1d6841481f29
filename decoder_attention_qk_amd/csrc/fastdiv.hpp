// Division of 31-bit unsigned values by a fixed divisor with one multiply-high
// (Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994): q = (mulhi(n, m) + n) >> l with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1.  Exact for n < 2^31 and 1 <= d < 2^31
// (the sum mulhi + n then stays below 2^32).  Host-compilable without HIP.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define MUSE_HD __host__ __device__
#else
#define MUSE_HD
#endif

namespace muse {

struct FastDiv {
  uint32_t d, m, l;
  FastDiv() : d(1), m(1), l(0) {}
  explicit FastDiv(uint32_t div) : d(div) {
    l = 0;
    while ((1ull << l) < div) ++l;
    m = (uint32_t)(((1ull << 32) * ((1ull << l) - div)) / div + 1);
  }
  MUSE_HD inline uint32_t div(uint32_t n) const {
#if defined(__HIP_DEVICE_COMPILE__)
    const uint32_t t = __umulhi(n, m);
#else
    const uint32_t t = (uint32_t)(((uint64_t)n * m) >> 32);
#endif
    return (t + n) >> l;
  }
  MUSE_HD inline uint32_t mod(uint32_t n) const { return n - div(n) * d; }
};

}  // namespace muse
