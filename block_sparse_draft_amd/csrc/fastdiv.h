// Division by a runtime constant through a precomputed multiplier, for the
// row-index arithmetic of the kernels (packed row -> draft block, head, token).
//
// For 1 <= d < 2^31 and 0 <= n < 2^31:  l = ceil(log2 d),
// m = floor(2^32 * (2^l - d) / d) + 1,  n / d = (mulhi(n, m) + n) >> l
// (Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994).  mulhi(n, m) <= n, so the sum stays below 2^32.
#pragma once
#include <stdint.h>

namespace skv {

struct FastDiv {
  uint32_t m, l;
  int32_t d;

  static FastDiv make(int32_t d) {
    FastDiv f;
    f.d = d;
    uint32_t l = 0;
    while ((1ull << l) < (uint64_t)d) ++l;
    f.l = l;
    f.m = (uint32_t)((((1ull << l) - (uint64_t)d) << 32) / (uint64_t)d + 1);
    return f;
  }
  __host__ __device__ inline int32_t div(int32_t n) const {
    const uint32_t t = (uint32_t)(((uint64_t)(uint32_t)n * m) >> 32);
    return (int32_t)((t + (uint32_t)n) >> l);
  }
  __host__ __device__ inline int32_t mod(int32_t n) const { return n - div(n) * d; }
};

}  // namespace skv
