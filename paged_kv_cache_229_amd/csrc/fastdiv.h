// Division by a divisor fixed for many uses, without a hardware divide (the work planner divides key
// counts by partition lengths many times per call; a 32-bit division is a long instruction sequence on
// this GPU and a 64-bit one a longer software routine).  Host and device code: the host build of
// tests/native/fastdiv_check.cpp checks it against integer division.
//
// For 2 <= d < 2^31 let m = floor((2^32 - 1) / d) + 1, so m d = 2^32 + e with 0 <= e < d.  For n < 2^32,
// n m / 2^32 = n / d + n e / (d 2^32), and the second term lies in [0, 1): q = floor(n m / 2^32) is
// floor(n / d) or one more, and q d > n tells the second case (q d < n + d <= 2^32 for n < 2^31, so the
// product does not wrap).
#pragma once

#include <stdint.h>

namespace pkv {

struct FastDiv {
  unsigned d, m;
  __host__ __device__ explicit FastDiv(int divisor)
      : d(static_cast<unsigned>(divisor)), m(0xffffffffu / static_cast<unsigned>(divisor) + 1u) {}
  // High half of the 64-bit product (one v_mul_hi_u32 on the device).
  __host__ __device__ static unsigned mulhi(unsigned a, unsigned b) {
    return static_cast<unsigned>((static_cast<uint64_t>(a) * b) >> 32);
  }
  // floor(n / d) for 0 <= n < 2^31.
  __host__ __device__ int floor_div(int n) const {
    unsigned q = mulhi(static_cast<unsigned>(n), m);
    q -= q * d > static_cast<unsigned>(n) ? 1u : 0u;
    return static_cast<int>(q);
  }
  // ceil(n / d) for 0 <= n < 2^31.
  __host__ __device__ int ceil_div(int n) const {
    const unsigned a = static_cast<unsigned>(n) + d - 1u;
    unsigned q = mulhi(a, m);
    q -= q * d > a ? 1u : 0u;
    return static_cast<int>(q);
  }
};

}  // namespace pkv
