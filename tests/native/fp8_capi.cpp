// Test-only C entry to the e4m3 encoder of the FP8 LM head (k_fp8.hpp), built
// with g++ on a machine without a GPU: the same source the weight conversion
// and the final norm compile for the device.
#include <cmath>
#include <cstdint>

#include "k_fp8.hpp"

// codes[i] = code of ldexp(x[i], -e[i]), the scaled value both conversions encode
extern "C" void svp_e4m3_codes(const float *x, const int32_t *e, uint32_t *codes, int64_t n) {
  for (int64_t i = 0; i < n; ++i) codes[i] = sv::e4m3_code(std::ldexp(x[i], -e[i]));
}

extern "C" void svp_e4m3_values(const uint32_t *codes, float *v, int64_t n) {
  for (int64_t i = 0; i < n; ++i) v[i] = sv::e4m3_value(codes[i]);
}

extern "C" void svp_fp8_exponents(const float *amax, int32_t *e, int64_t n) {
  for (int64_t i = 0; i < n; ++i) e[i] = sv::fp8_exponent(amax[i]);
}

extern "C" int svp_fp8_weight_ok(float w) { return sv::fp8_weight_ok(w) ? 1 : 0; }
