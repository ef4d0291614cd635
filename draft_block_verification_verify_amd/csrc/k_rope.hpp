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

// Workgroup (i, by) of ry workgroups of row i takes the row's (head, pair)
// items by * 256 + thread, then every ry * 256 further.  Each workgroup first
// builds the row's sine/cosine table (d/2 <= 128 entries) once, then rotates
// its items four at a time, every load of the four issued before the
// arithmetic.
template <typename T>
__device__ __forceinline__ void rope_rows_block(const T *__restrict__ q, const T *__restrict__ k,
                                                T *__restrict__ q_out, T *__restrict__ k_out,
                                                const int32_t *__restrict__ row_pos, int Hq, int Hkv, int D,
                                                double base, int64_t q_lo_off, int64_t k_lo_off, int i, int by,
                                                int ry) {
  __shared__ double cs[128], sn[128];   // cos, sin of pos * theta_k, k < D/2 <= 128
  const int half = D / 2;
  const int items = (Hq + Hkv) * half;
  const double pos = double(row_pos[i]);
  if (threadIdx.x < half) {
    const double theta = pow(base, -2.0 * double(threadIdx.x) / double(D));
    sincos(pos * theta, &sn[threadIdx.x], &cs[threadIdx.x]);
  }
  __syncthreads();
  const int stride = ry * blockDim.x;
  for (int p0 = by * blockDim.x + threadIdx.x; p0 < items; p0 += 4 * stride) {
    double a[4], b[4];
    const T *src[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = p0 + u * stride;
      const int hh = p < items ? p / half : 0, kk = p % half;
      src[u] = hh < Hq ? q + (int64_t(i) * Hq + hh) * D : k + (int64_t(i) * Hkv + (hh - Hq)) * D;
      a[u] = b[u] = 0.0;
      if (p < items) {
        a[u] = ld(src[u] + kk);
        b[u] = ld(src[u] + kk + half);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = p0 + u * stride;
      if (p >= items) continue;
      const int hh = p / half, kk = p % half;
      const double c = cs[kk], sv_ = sn[kk];
      if (hh < Hq) {
        T *dst = q_out + (int64_t(i) * Hq + hh) * D;
        st_q(dst + kk, q_lo_off, a[u] * c - b[u] * sv_);
        st_q(dst + kk + half, q_lo_off, b[u] * c + a[u] * sv_);
      } else {
        T *dst = k_out + (int64_t(i) * Hkv + (hh - Hq)) * D;
        st_q(dst + kk, k_lo_off, a[u] * c - b[u] * sv_);
        st_q(dst + kk + half, k_lo_off, b[u] * c + a[u] * sv_);
      }
    }
  }
}

}  // namespace sv
