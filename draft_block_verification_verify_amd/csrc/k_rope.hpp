// RoPE of the verify rows (device code shared by the attention file and the
// launch that runs it beside the drafter statistics).
#pragma once
#include "k_common.hpp"

namespace sv {

// ----------------------------------------------------------------------------
// RoPE of the row queries and keys at their semantic positions: pair k couples
// components k and k + d/2 and turns by pos * base^(-2k/d).  Angles, sines and
// cosines in fp64; the rotated values are rounded once to the output type.
// ----------------------------------------------------------------------------

template <typename T>
__device__ __forceinline__ double ld(const T *p);
template <>
__device__ __forceinline__ double ld<uint16_t>(const uint16_t *p) { return double(bf2f(*p)); }
template <>
__device__ __forceinline__ double ld<float>(const float *p) { return double(*p); }

// bf16 queries (and keys) are written as a hi plane (q_out) and a lo plane
// (q_out + lo_off) with hi + lo = rotated value to about 16 bits.  The key's
// hi plane is the key rounded to bf16 once, as a cache entry holds it.
__device__ __forceinline__ void st_q(uint16_t *p, int64_t lo_off, double v) {
  uint16_t hi, lo;
  split_bf(float(v), hi, lo);
  p[0] = hi;
  p[lo_off] = lo;
}
__device__ __forceinline__ void st_q(float *p, int64_t, double v) { *p = float(v); }

// One thread per (row, head, pair): workgroup (i, by) of 256 threads takes
// pairs by * 256 + thread of row i.  Each workgroup first builds the row's sine/cosine table (d/2 <= 128
// entries), so every thread then does one load pair, one rotation and one
// store pair, with no chain of dependent memory accesses.
template <typename T>
__device__ __forceinline__ void rope_rows_block(const T *__restrict__ q, const T *__restrict__ k,
                                                T *__restrict__ q_out, T *__restrict__ k_out,
                                                const int32_t *__restrict__ row_pos, int Hq, int Hkv, int D,
                                                double base, int64_t q_lo_off, int64_t k_lo_off, int i, int by) {
  __shared__ double cs[128], sn[128];   // cos, sin of pos * theta_k, k < D/2 <= 128
  const int half = D / 2;
  const int heads = Hq + Hkv;
  const int p = by * blockDim.x + threadIdx.x;
  const bool active = p < heads * half;
  const int hh = active ? p / half : 0, kk = p % half;
  // issue this thread's loads before the table's arithmetic
  const T *src = hh < Hq ? q + (int64_t(i) * Hq + hh) * D : k + (int64_t(i) * Hkv + (hh - Hq)) * D;
  double a = 0.0, b = 0.0;
  if (active) {
    a = ld(src + kk);
    b = ld(src + kk + half);
  }
  const double pos = double(row_pos[i]);
  if (threadIdx.x < half) {
    const double theta = pow(base, -2.0 * double(threadIdx.x) / double(D));
    sincos(pos * theta, &sn[threadIdx.x], &cs[threadIdx.x]);
  }
  __syncthreads();
  if (!active) return;
  const double c = cs[kk], s = sn[kk];
  if (hh < Hq) {
    T *dst = q_out + (int64_t(i) * Hq + hh) * D;
    st_q(dst + kk, q_lo_off, a * c - b * s);
    st_q(dst + kk + half, q_lo_off, b * c + a * s);
  } else {
    T *dst = k_out + (int64_t(i) * Hkv + (hh - Hq)) * D;
    st_q(dst + kk, k_lo_off, a * c - b * s);
    st_q(dst + kk + half, k_lo_off, b * c + a * s);
  }
}

}  // namespace sv
