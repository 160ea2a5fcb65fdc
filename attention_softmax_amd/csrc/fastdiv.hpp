// fastdiv.hpp -- unsigned 32-bit division by a divisor fixed at launch time,
// as one high multiply, one add and one shift.
//
// Method: T. Granlund and P. L. Montgomery, "Division by Invariant Integers
// using Multiplication" (PLDI 1994), the round-up variant for unsigned N-bit
// operands: with l = ceil(log2 d) and m = floor(2^N (2^l - d) / d) + 1 (which
// fits in N bits), n / d = (mulhi(m, n) + n) >> l for every 0 <= n < 2^N. The
// sum is formed in 64 bits, so it cannot overflow.
//
// Plain C++ (host) and HIP (device); tests/test_fastdiv.py compiles this header
// with g++ and checks it against '/' on edge and random operands.

#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define SMS_HD __host__ __device__ __forceinline__
#else
#define SMS_HD inline
#endif

namespace sms {

struct FastDiv {
  uint32_t d;  // divisor (>= 1)
  uint32_t m;  // magic multiplier
  uint32_t l;  // shift, ceil(log2 d)
};

inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t l = 0;
  while (l < 32 && (uint64_t(1) << l) < d) ++l;
  f.l = l;
  f.m = (uint32_t)(((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1);
  return f;
}

SMS_HD uint32_t mulhi32(uint32_t a, uint32_t b) {
  return (uint32_t)(((uint64_t)a * (uint64_t)b) >> 32);
}

SMS_HD uint32_t fast_div(uint32_t n, const FastDiv& f) {
  return (uint32_t)(((uint64_t)mulhi32(f.m, n) + n) >> f.l);
}

}  // namespace sms
