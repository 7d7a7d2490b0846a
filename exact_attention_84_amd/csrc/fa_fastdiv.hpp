// Division of non-negative integers below 2^31 by a divisor that is fixed for
// a launch (head counts, tiles per head): a multiply-high, an add and a
// shift, by the round-up method of division by invariant integers (Granlund
// and Montgomery, "Division by invariant integers using multiplication",
// 1994).  With l = ceil(log2 d) and m = ceil(2^(32+l) / d) - 2^32,
//   floor(n / d) = floor((n + floor(m n / 2^32)) / 2^l)   for 0 <= n < 2^32,
// and n < 2^31 keeps the sum inside 32 bits.  The host computes m and l once;
// device code then divides with scalar multiplies instead of the reciprocal
// sequence a runtime divisor otherwise costs.  Host and device code, no
// intrinsics, so that a host test can check it.
#pragma once

#include <cstdint>

#if defined(__HIPCC__)
#define FA_FD __host__ __device__ __forceinline__
#else
#define FA_FD inline
#endif

namespace fa {

struct FastDiv {
  uint32_t d;  // divisor, 1 <= d < 2^31
  uint32_t m;  // ceil(2^(32+l) / d) - 2^32 (1 for a power of two, which gives the same quotients)
  uint32_t l;  // ceil(log2 d)

  static FA_FD FastDiv make(uint32_t d) {
    FastDiv f{d, 0u, 0u};
    while ((1ull << f.l) < d) ++f.l;
    f.m = static_cast<uint32_t>(((1ull << 32) * ((1ull << f.l) - d)) / d + 1);
    return f;
  }
  // floor(n / d) for 0 <= n < 2^31
  FA_FD uint32_t div(uint32_t n) const {
    const uint32_t t = static_cast<uint32_t>((static_cast<uint64_t>(m) * n) >> 32);
    return (t + n) >> l;
  }
};

}  // namespace fa
