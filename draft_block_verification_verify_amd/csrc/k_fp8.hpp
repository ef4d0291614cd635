// OCP e4m3 encoding of the FP8 LM head: 4 exponent bits (bias 7), 3 mantissa
// bits, largest finite 448, subnormal step 2^-9, no infinities; values are
// rounded to the nearest code, ties to even.  Row scales are powers of two.
//
// Plain C++ arithmetic on floats and integers, compiled for the GPU (the
// weight conversion and the final norm) and by g++ for the CPU tests that
// compare every code with a brute-force nearest-value search.
#pragma once

#include <cmath>
#include <cstdint>

#if defined(__HIPCC__)
#define SV_HD __host__ __device__
#else
#define SV_HD
#endif

namespace sv {

SV_HD inline uint32_t fp8_bits(float x) { return __builtin_bit_cast(uint32_t, x); }
SV_HD inline float fp8_float(uint32_t u) { return __builtin_bit_cast(float, u); }

// Sign and magnitude code of x, |x| <= 448 (a larger |x| saturates at the
// largest finite code, 0x7E; NaN gives the NaN code 0x7F).
SV_HD inline uint32_t e4m3_code(float x) {
  const uint32_t u = fp8_bits(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = std::fabs(x);
  if (!(a <= 448.0f)) return sign | (a > 448.0f ? 0x7Eu : 0x7Fu);
  uint32_t code;
  if (a < 0.015625f) {
    // below 2^-6: multiples of 2^-9 (the product is exact; rint rounds half to even)
    code = uint32_t(std::rint(a * 512.0f));
  } else {
    // keep 3 mantissa bits, rounding the 20 dropped bits half to even
    const uint32_t b = fp8_bits(a);
    const uint32_t r = (b + 0x7FFFFu + ((b >> 20) & 1u)) & ~0xFFFFFu;
    const int e = int(r >> 23) - 127;
    code = (uint32_t(e + 7) << 3) | ((r >> 20) & 7u);
  }
  return sign | code;
}

// Value of a code (for the tests; 0x7F / 0xFF is NaN).
SV_HD inline float e4m3_value(uint32_t code) {
  const uint32_t e = (code >> 3) & 15u, m = code & 7u;
  if ((code & 0x7Fu) == 0x7Fu) return NAN;
  const float v = e == 0 ? float(m) * 0.001953125f : std::ldexp(1.0f + float(m) * 0.125f, int(e) - 7);
  return (code & 0x80u) ? -v : v;
}

// Smallest scale exponent e, at least -126 (so that 2^e is a normal float),
// with amax <= 448 * 2^e; 0 for amax == 0 or a value that is not finite.
// With amax = f 2^k, f in [0.5, 1), and 448 = 0.875 * 2^9: e = k - 9 when
// f <= 0.875, else k - 8.  No loop, no division.
SV_HD inline int fp8_exponent(float amax) {
  if (!(amax > 0.0f) || !(amax <= 3.4028234663852886e38f)) return 0;
  int k = 0;
  const float f = std::frexp(amax, &k);
  const int e = k - 9 + (f > 0.875f ? 1 : 0);
  return e < -126 ? -126 : e;
}

// Whether a weight can be quantised: finite.
SV_HD inline bool fp8_weight_ok(float w) { return std::fabs(w) <= 3.4028234663852886e38f; }

}  // namespace sv
