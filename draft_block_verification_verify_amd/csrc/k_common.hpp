// Device-side helpers shared by the gfx950 kernels: bf16 bit handling, MFMA
// wrappers, wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.hpp"

namespace sv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return uint32_t(f2bf(lo)) | (uint32_t(f2bf(hi)) << 16);
}

__device__ __forceinline__ bf16x8 as_bf8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load marked non-temporal (streamed data that is read once).
__device__ __forceinline__ uint4 ld_nt16(const void *p) {
  const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// fp32 -> fp16 bits, round to nearest even.
__device__ __forceinline__ uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f)); }

__device__ __forceinline__ float h2f(uint16_t b) { return float(__builtin_bit_cast(_Float16, b)); }

// Split x into fp16 hi + lo with hi + lo = x to about 22 significant bits.
__device__ __forceinline__ void split_h(float x, uint16_t &hi, uint16_t &lo) {
  hi = f2h(x);
  lo = f2h(x - h2f(hi));
}

// Split x into bf16 hi + lo with hi + lo = x to about 16 significant bits.
__device__ __forceinline__ void split_bf(float x, uint16_t &hi, uint16_t &lo) {
  hi = f2bf(x);
  lo = f2bf(x - bf2f(hi));
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 in one word (x in the low half), round to nearest
// even, by the gfx950 packed conversion instruction.
__device__ __forceinline__ uint32_t cvt_bf2(float x, float y) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x, y}, bf16x2_t));
}

// hi + lo split of two values at once: hi = bf16(v), lo = bf16(v - hi),
// each pair packed as cvt_bf2 packs it.
__device__ __forceinline__ void split_bf2(float x, float y, uint32_t &hi, uint32_t &lo) {
  hi = cvt_bf2(x, y);
  lo = cvt_bf2(x - __uint_as_float(hi << 16), y - __uint_as_float(hi & 0xFFFF0000u));
}

// 8 bf16 -> 8 fp16, round to nearest even.  Exact for 0 and for 2^-17 <=
// |x| <= 65504 (a bf16 significand has 8 bits, so its last bit is at least
// 2^-24, fp16's subnormal step, from 2^-17 up); smaller magnitudes become the
// nearest multiple of 2^-24.
__device__ __forceinline__ uint4 bf8_to_h8(uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __uint_as_float(w[i] << 16), hi = __uint_as_float(w[i] & 0xFFFF0000u);
    o[i] = uint32_t(f2h(lo)) | (uint32_t(f2h(hi)) << 16);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// A weight the fp16 copy cannot hold: |w| > 65504, infinite or NaN.
__device__ __forceinline__ int not_f16(float w) { return !(fabsf(w) <= 65504.f); }

// D(32x32) += A(32x16) * B(16x32).  Lane l supplies A[l%32][8*(l/32)+0..7],
// B[8*(l/32)+0..7][l%32]; acc element j of lane l is
// D[8*(j/4) + 4*(l/32) + (j%4)][l%32].
__device__ __forceinline__ f32x16 mfma32(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(a), as_bf8(b), c, 0, 0, 0);
}

// Same layout with fp16 operands.
__device__ __forceinline__ f32x16 mfma32h(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                0);
}

// D(16x16) += A(16x32) * B(32x16).  Lane l supplies A[l%16][8*(l/16)+0..7],
// B[8*(l/16)+0..7][l%16]; acc element i of lane l is D[4*(l/16) + i][l%16].
__device__ __forceinline__ f32x4 mfma16(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(a), as_bf8(b), c, 0, 0, 0);
}

// Whole-wavefront reductions on DPP moves (a permute butterfly of
// __shfl_xor compiles to six LDS round trips): xor 1 and xor 2 inside each
// quad, the half-row and row mirrors (8 and 16 lanes), then the row
// broadcasts of lane 15 and lane 31 carry the partial results up to lane 63,
// which every lane then reads.  Every lane of the wavefront must be active.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_move(float v, float fill) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(fill), __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}

__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_move<0xB1>(v, 0.f);         // quad_perm [1,0,3,2]
  v += dpp_move<0x4E>(v, 0.f);         // quad_perm [2,3,0,1]
  v += dpp_move<0x141>(v, 0.f);        // row_half_mirror
  v += dpp_move<0x140>(v, 0.f);        // row_mirror
  v += dpp_move<0x142, 0xA>(v, 0.f);   // row_bcast15 into rows 1 and 3
  v += dpp_move<0x143, 0xC>(v, 0.f);   // row_bcast31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_move<0xB1>(v, -INFINITY));
  v = fmaxf(v, dpp_move<0x4E>(v, -INFINITY));
  v = fmaxf(v, dpp_move<0x141>(v, -INFINITY));
  v = fmaxf(v, dpp_move<0x140>(v, -INFINITY));
  v = fmaxf(v, dpp_move<0x142, 0xA>(v, -INFINITY));
  v = fmaxf(v, dpp_move<0x143, 0xC>(v, -INFINITY));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float wave_max(float v) { return wave_max_dpp(v); }
__device__ __forceinline__ float wave_sum(float v) { return wave_sum_dpp(v); }

// Reductions over the four lanes l, l^16, l^32, l^48 (one per 16-lane row)
// with the gfx950 row swaps: v_permlane16_swap exchanges the odd rows of its
// first operand with the even rows of its second, v_permlane32_swap the upper
// half of the first with the lower half of the second; with both operands
// equal, the two results of a swap hold every lane's partner of that step.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float rows4_max(float v) {
  u32x2 r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r.x), __uint_as_float(r.y));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r.x), __uint_as_float(r.y));
}

__device__ __forceinline__ float rows4_sum(float v) {
  u32x2 r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r.x) + __uint_as_float(r.y);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r.x) + __uint_as_float(r.y);
}

// Running (max, sum of exp(x - max), index of the max) of a set of logits.
// The index is the lowest among equal maxima.
struct MaxSumArg {
  float m, s;
  int i;
};

__device__ __forceinline__ MaxSumArg msa_empty() { return {-INFINITY, 0.f, 0x7fffffff}; }

__device__ __forceinline__ MaxSumArg msa_merge(MaxSumArg a, MaxSumArg b) {
  MaxSumArg r;
  r.m = fmaxf(a.m, b.m);
  if (r.m == -INFINITY) {
    r.s = 0.f;
  } else {
    r.s = a.s * __expf(a.m - r.m) + b.s * __expf(b.m - r.m);
  }
  r.i = (b.m > a.m || (b.m == a.m && b.i < a.i)) ? b.i : a.i;
  return r;
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ MaxSumArg msa_dpp_step(MaxSumArg a) {
  const MaxSumArg e = msa_empty();
  MaxSumArg b;
  b.m = dpp_move<CTRL, ROW_MASK>(a.m, e.m);
  b.s = dpp_move<CTRL, ROW_MASK>(a.s, e.s);
  b.i = __builtin_amdgcn_update_dpp(e.i, a.i, CTRL, ROW_MASK, 0xF, false);
  return msa_merge(a, b);
}

// (max, sum exp, argmax) over the wavefront (the DPP sequence of wave_sum);
// every lane gets lane 63's result
__device__ __forceinline__ MaxSumArg msa_wave(MaxSumArg r) {
  r = msa_dpp_step<0xB1>(r);
  r = msa_dpp_step<0x4E>(r);
  r = msa_dpp_step<0x141>(r);
  r = msa_dpp_step<0x140>(r);
  r = msa_dpp_step<0x142, 0xA>(r);
  r = msa_dpp_step<0x143, 0xC>(r);
  return MaxSumArg{__int_as_float(__builtin_amdgcn_readlane(__float_as_int(r.m), 63)),
                   __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r.s), 63)),
                   __builtin_amdgcn_readlane(r.i, 63)};
}

__device__ __forceinline__ MaxSumArg msa_shfl_xor(MaxSumArg a, int mask) {
  MaxSumArg b;
  b.m = __shfl_xor(a.m, mask);
  b.s = __shfl_xor(a.s, mask);
  b.i = __shfl_xor(a.i, mask);
  return msa_merge(a, b);
}

}  // namespace sv
