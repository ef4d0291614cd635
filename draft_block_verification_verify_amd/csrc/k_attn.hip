// Rotary positions and tree-masked GQA attention for the verify step (gfx950).
//
// Rows attend to their tree's KV prefix plus their ancestors and themselves,
// with RoPE at the rows' semantic positions (onedev.kr SpecOPD summary,
// "what differs": parent map, semantic positions, ancestor-and-self mask).
//
// bf16 path: split-KV flash-decode.  A work item is (tree, KV head, query
// group, key range); its query vectors are the tree's (row, head-in-group)
// pairs, so one K/V tile streamed from HBM serves every row and every query
// head of the GQA group.  K/V tiles of 32 keys are staged through LDS (V
// transposed on the way in), S^T = K.Q^T and O^T += V^T.P^T run on
// 16x16x32 bf16 MFMA, the online softmax is per wavefront in fp32 (log2
// domain).  The rotated queries and the probabilities are each carried as a
// bf16 pair hi + lo (two MFMAs per product), so the only bf16 rounding left
// in the scores is the one of the cached keys themselves.  Each item leaves
// (max, sum, unnormalised o) per query; a merge kernel combines the items of
// a query and writes o in the format the W_o projection reads.
//
// fp32 path: one workgroup per (row, query head), plain fp32 arithmetic.
#include "k_common.hpp"
#include "launch.hpp"

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

template <typename T>
__device__ __forceinline__ void st(T *p, double v);
template <>
__device__ __forceinline__ void st<uint16_t>(uint16_t *p, double v) { *p = f2bf(float(v)); }
template <>
__device__ __forceinline__ void st<float>(float *p, double v) { *p = float(v); }

// bf16 queries are written as a hi plane (q_out) and a lo plane
// (q_out + q_lo_off) with hi + lo = rotated value to about 16 bits.
__device__ __forceinline__ void st_q(uint16_t *p, int64_t lo_off, double v) {
  uint16_t hi, lo;
  split_bf(float(v), hi, lo);
  p[0] = hi;
  p[lo_off] = lo;
}
__device__ __forceinline__ void st_q(float *p, int64_t, double v) { *p = float(v); }

template <typename T>
__global__ __launch_bounds__(256) void rope_rows_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                        T *__restrict__ q_out, T *__restrict__ k_out,
                                                        const int32_t *__restrict__ row_pos, int Hq,
                                                        int Hkv, int D, double base, int64_t q_lo_off) {
  const int i = blockIdx.x;
  const int half = D / 2;
  const int heads = Hq + Hkv;
  const double pos = double(row_pos[i]);
  for (int p = threadIdx.x; p < heads * half; p += blockDim.x) {
    const int hh = p / half, kk = p % half;
    const T *src;
    T *dst;
    if (hh < Hq) {
      src = q + (int64_t(i) * Hq + hh) * D;
      dst = q_out + (int64_t(i) * Hq + hh) * D;
    } else {
      src = k + (int64_t(i) * Hkv + (hh - Hq)) * D;
      dst = k_out + (int64_t(i) * Hkv + (hh - Hq)) * D;
    }
    const double theta = pow(base, -2.0 * double(kk) / double(D));
    double s, c;
    sincos(pos * theta, &s, &c);
    const double a = ld(src + kk), b = ld(src + kk + half);
    if (hh < Hq) {
      st_q(dst + kk, q_lo_off, a * c - b * s);
      st_q(dst + kk + half, q_lo_off, b * c + a * s);
    } else {
      st(dst + kk, a * c - b * s);
      st(dst + kk + half, b * c + a * s);
    }
  }
}

// ----------------------------------------------------------------------------
// bf16 split-KV attention on MFMA
// ----------------------------------------------------------------------------

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void attn_mfma_kernel(AttnArgs a) {
  constexpr int NT = 64 * NW;     // threads
  constexpr int KT = 32;          // keys per LDS tile
  constexpr int KROW = D + 8;     // bf16 per LDS K row (16 B pad: conflict-free b128 reads)
  constexpr int VROW = KT + 4;    // bf16 per LDS V^T row (72 B)
  constexpr int DS = D / 32;      // 32-wide d steps of S = K.Q^T
  constexpr int DB = D / 16;      // 16-wide d blocks of O^T
  constexpr int KUN = KT * D / 8;                      // 16-B K chunks per tile
  constexpr int KCH = (KUN + NT - 1) / NT;
  constexpr int VUN = (KT / 2) * (D / 8);              // (key pair, 16-B column) units
  constexpr int VCH = (VUN + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][KT * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][D * VROW];

  const AttnItem it = a.items[blockIdx.x];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n16 = lane & 15, kg = lane >> 4;
  const int r = it.tree;
  const int s0 = a.tree_start[r], T = a.tree_rows[r], klen = a.tree_kv_len[r];
  const int64_t koff = a.tree_kv_off[r];
  const int g = it.g, G = a.G, Hkv = a.Hkv, Hq = a.Hq;
  const int nkeys = klen + T;
  const int QB = (it.nq + 15) / 16;   // <= NW
  const bool wave_on = w < QB;

  // ---- this wave's query fragments (B operand of S^T = K.Q^T), hi and lo
  uint4 qh[DS], ql[DS];
  const int mq = w * 16 + n16;
  const bool qok = wave_on && mq < it.nq;
  uint64_t anc = 0;
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) qh[ds] = ql[ds] = make_uint4(0, 0, 0, 0);
  if (qok) {
    const int m = it.m0 + mq;
    const int row = s0 + m / G;
    const int head = g * G + m % G;
    const uint16_t *qp = a.q_rot + (int64_t(row) * Hq + head) * D + kg * 8;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      qh[ds] = *reinterpret_cast<const uint4 *>(qp + ds * 32);
      ql[ds] = *reinterpret_cast<const uint4 *>(qp + a.q_lo_off + ds * 32);
    }
    anc = a.row_anc[row];
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- staging registers for one tile
  uint4 kreg[KCH];
  uint4 vreg[VCH][2];
  auto key_src = [&](int v, const uint16_t *pre, const uint16_t *rows) -> const uint16_t * {
    if (v < klen) return pre + ((koff + v) * Hkv + g) * int64_t(D);
    if (v < nkeys) return rows + (int64_t(s0 + v - klen) * Hkv + g) * D;
    return nullptr;
  };
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      const int c = tid + NT * j;
      const int kk = c / (D / 8), col = c % (D / 8);
      const uint16_t *p = (c < KUN) ? key_src(kt + kk, a.kv_k, a.k_rot) : nullptr;
      kreg[j] = p ? *reinterpret_cast<const uint4 *>(p + col * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < VCH; ++j) {
      const int u = tid + NT * j;
      const int pr = u % (KT / 2), col = u / (KT / 2);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const uint16_t *p = (u < VUN) ? key_src(kt + 2 * pr + e, a.kv_v, a.v_rows) : nullptr;
        vreg[j][e] = p ? *reinterpret_cast<const uint4 *>(p + col * 8) : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&](int b) {
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      const int c = tid + NT * j;
      if (c < KUN) {
        const int kk = c / (D / 8), col = c % (D / 8);
        *reinterpret_cast<uint4 *>(&k_lds[b][kk * KROW + col * 8]) = kreg[j];
      }
    }
#pragma unroll
    for (int j = 0; j < VCH; ++j) {
      const int u = tid + NT * j;
      if (u < VUN) {
        const int pr = u % (KT / 2), col = u / (KT / 2);
        const uint32_t *w0 = reinterpret_cast<const uint32_t *>(&vreg[j][0]);
        const uint32_t *w1 = reinterpret_cast<const uint32_t *>(&vreg[j][1]);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const uint32_t lo = (w0[t >> 1] >> (16 * (t & 1))) & 0xFFFFu;
          const uint32_t hi = (w1[t >> 1] >> (16 * (t & 1))) & 0xFFFFu;
          *reinterpret_cast<uint32_t *>(&v_lds[b][(col * 8 + t) * VROW + 2 * pr]) = lo | (hi << 16);
        }
      }
    }
  };

  const int nsub = (it.k1 - it.k0 + KT - 1) / KT;
  load_tile(it.k0);
  store_tile(0);
  __syncthreads();
  for (int stp = 0; stp < nsub; ++stp) {
    const int b = stp & 1;
    const int kt = it.k0 + stp * KT;
    if (stp + 1 < nsub) load_tile(kt + KT);
    if (wave_on) {
      // S^T = K.(Q_hi + Q_lo)^T for two 16-key blocks
      f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const uint4 kf = *reinterpret_cast<const uint4 *>(&k_lds[b][(16 * kb + n16) * KROW + ds * 32 + kg * 8]);
          sacc[kb] = mfma16(kf, qh[ds], sacc[kb]);
          sacc[kb] = mfma16(kf, ql[ds], sacc[kb]);
        }
      }
      // masked online softmax (log2 domain) for the lane's query
      float x[2][4];
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int v = kt + 16 * kb + 4 * kg + i;
          const bool ok = qok && v < it.k1 && (v < klen || ((anc >> (v - klen)) & 1ull));
          x[kb][i] = ok ? sacc[kb][i] * a.scale_log2 : -INFINITY;
          tmax = fmaxf(tmax, x[kb][i]);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float m_new = fmaxf(m_run, tmax);
      const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2f(m_run - m_ref);
      float p[2][4];
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[kb][i] = exp2f(x[kb][i] - m_ref);
          rs += p[kb][i];
        }
      rs += __shfl_xor(rs, 16);
      rs += __shfl_xor(rs, 32);
      l_run = l_run * alpha + rs;
      m_run = m_new;
      // P as hi + lo bf16 pairs; key slot 8*kg + t <-> key 4*kg + t (t < 4),
      // 16 + 4*kg + t - 4 (t >= 4), the same order the V^T fragments use
      uint16_t ph[2][4], pl[2][4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) split_bf(p[kb][i], ph[kb][i], pl[kb][i]);
      const uint4 pfh = make_uint4(ph[0][0] | (uint32_t(ph[0][1]) << 16), ph[0][2] | (uint32_t(ph[0][3]) << 16),
                                   ph[1][0] | (uint32_t(ph[1][1]) << 16), ph[1][2] | (uint32_t(ph[1][3]) << 16));
      const uint4 pfl = make_uint4(pl[0][0] | (uint32_t(pl[0][1]) << 16), pl[0][2] | (uint32_t(pl[0][3]) << 16),
                                   pl[1][0] | (uint32_t(pl[1][1]) << 16), pl[1][2] | (uint32_t(pl[1][3]) << 16));
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint16_t *vrow = &v_lds[b][(db * 16 + n16) * VROW];
        const uint2 lo = *reinterpret_cast<const uint2 *>(vrow + 4 * kg);
        const uint2 hi = *reinterpret_cast<const uint2 *>(vrow + 16 + 4 * kg);
        const uint4 vf = make_uint4(lo.x, lo.y, hi.x, hi.y);
        o[db] = o[db] * alpha;
        o[db] = mfma16(vf, pfh, o[db]);
        o[db] = mfma16(vf, pfl, o[db]);
      }
    }
    if (stp + 1 < nsub) store_tile(b ^ 1);
    __syncthreads();
  }

  // ---- partial results
  if (qok) {
    const int64_t slot = int64_t(it.slot) + mq;
    if (kg == 0) {
      a.part_ml[2 * slot] = m_run;
      a.part_ml[2 * slot + 1] = l_run;
    }
    float *po = a.part_o + slot * D + 4 * kg;
#pragma unroll
    for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4 *>(po + db * 16) = o[db];
  }
}

// Combine the split-KV partials of one (row, query head) and write o (bf16).
template <int D>
__global__ __launch_bounds__(D) void attn_merge_kernel(MergeArgs a) {
  const int i = blockIdx.x / a.Hq, h = blockIdx.x % a.Hq;
  const int G = a.Hq / a.Hkv;
  const int r = a.row_tree[i], loc = a.row_local[i];
  const int g = h / G, m = loc * G + h % G;
  const int qg = m / kItemQ, mi = m % kItemQ;
  const int gi = (r * a.Hkv + g) * a.qg_max + qg;
  const int first = a.group_first[gi], cnt = a.group_count[gi];
  float M = -INFINITY;
  for (int t = 0; t < cnt; ++t) {
    const int64_t slot = int64_t(a.items[first + t].slot) + mi;
    M = fmaxf(M, a.part_ml[2 * slot]);
  }
  float L = 0.f, acc = 0.f;
  const int c = threadIdx.x;
  for (int t = 0; t < cnt; ++t) {
    const int64_t slot = int64_t(a.items[first + t].slot) + mi;
    const float mt = a.part_ml[2 * slot];
    const float wgt = (mt == -INFINITY) ? 0.f : exp2f(mt - M);
    L += wgt * a.part_ml[2 * slot + 1];
    acc += wgt * a.part_o[slot * D + c];
  }
  const float val = acc / L;
  const int64_t idx = int64_t(i) * a.Hq * D + int64_t(h) * D + c;
  if (a.mode == ACT_SPLIT) {
    uint16_t hi, lo;
    split_h(val, hi, lo);
    a.out[idx] = hi;
    a.out[a.lo_off + idx] = lo;
  } else {
    a.out[idx] = f2h(val);
  }
}

// ----------------------------------------------------------------------------
// fp32 attention: one workgroup per (row, query head), keys in tiles of 256.
// ----------------------------------------------------------------------------

__device__ __forceinline__ float block_max256(float v, float *red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ __forceinline__ float block_sum256(float v, float *red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ __launch_bounds__(256) void attn_f32_kernel(AttnF32Args a) {
  __shared__ float q_s[256];
  __shared__ float p_s[256];
  __shared__ float red[4];
  const int i = blockIdx.x / a.Hq, h = blockIdx.x % a.Hq;
  const int D = a.D, tid = threadIdx.x;
  const int G = a.Hq / a.Hkv, g = h / G;
  const int r = a.row_tree[i];
  const int s0 = a.tree_start[r], T = a.tree_rows[r], klen = a.tree_kv_len[r];
  const int64_t koff = a.tree_kv_off[r];
  const uint64_t anc = a.row_anc[i];
  const int nk = klen + T;
  if (tid < D) q_s[tid] = a.q_rot[(int64_t(i) * a.Hq + h) * D + tid];
  __syncthreads();
  auto kptr = [&](int v, const float *pre, const float *rows) -> const float * {
    return v < klen ? pre + ((koff + v) * a.Hkv + g) * int64_t(D)
                    : rows + (int64_t(s0 + v - klen) * a.Hkv + g) * D;
  };
  const float scale = 1.0f / sqrtf(float(D));
  float m_run = -INFINITY, l_run = 0.f, acc = 0.f;
  for (int kt = 0; kt < nk; kt += 256) {
    const int v = kt + tid;
    float x = -INFINITY;
    if (v < nk && (v < klen || ((anc >> (v - klen)) & 1ull))) {
      const float *kp = kptr(v, a.kv_k, a.k_rot);
      float s = 0.f;
      for (int c = 0; c < D; ++c) s = fmaf(q_s[c], kp[c], s);
      x = s * scale;
    }
    const float tmax = block_max256(x, red);
    const float m_new = fmaxf(m_run, tmax);
    const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = expf(m_run - m_ref);
    const float p = expf(x - m_ref);
    p_s[tid] = p;
    const float rs = block_sum256(p, red);
    l_run = l_run * alpha + rs;
    m_run = m_new;
    if (tid < D) {
      acc *= alpha;
      const int lim = min(256, nk - kt);
      for (int j = 0; j < lim; ++j) {
        const float pj = p_s[j];
        if (pj != 0.f) acc = fmaf(pj, kptr(kt + j, a.kv_v, a.v_rows)[tid], acc);
      }
    }
    __syncthreads();
  }
  if (tid < D) a.out[int64_t(i) * a.Hq * D + int64_t(h) * D + tid] = acc / l_run;
}

// ----------------------------------------------------------------------------
// launchers
// ----------------------------------------------------------------------------

void launch_rope_bf16(const uint16_t *q, const uint16_t *k, uint16_t *qo, uint16_t *ko, const int32_t *row_pos,
                      int n, int Hq, int Hkv, int D, double base, int64_t q_lo_off, hipStream_t s) {
  hipLaunchKernelGGL(rope_rows_kernel<uint16_t>, dim3(n), dim3(256), 0, s, q, k, qo, ko, row_pos, Hq, Hkv, D, base,
                     q_lo_off);
}

void launch_rope_f32(const float *q, const float *k, float *qo, float *ko, const int32_t *row_pos, int n, int Hq,
                     int Hkv, int D, double base, hipStream_t s) {
  hipLaunchKernelGGL(rope_rows_kernel<float>, dim3(n), dim3(256), 0, s, q, k, qo, ko, row_pos, Hq, Hkv, D, base,
                     int64_t(0));
}

void launch_attn_mfma(const AttnArgs &a, int n_items, int D, int max_qblocks, hipStream_t s) {
  const bool eight = max_qblocks > 4;
#define SV_ATTN(DD)                                                                              \
  if (D == DD) {                                                                                 \
    if (eight)                                                                                   \
      hipLaunchKernelGGL((attn_mfma_kernel<DD, 8>), dim3(n_items), dim3(512), 0, s, a);          \
    else                                                                                         \
      hipLaunchKernelGGL((attn_mfma_kernel<DD, 4>), dim3(n_items), dim3(256), 0, s, a);          \
    return;                                                                                      \
  }
  SV_ATTN(64)
  SV_ATTN(128)
  SV_ATTN(256)
#undef SV_ATTN
}

void launch_attn_merge(const MergeArgs &a, int n_rows, int D, hipStream_t s) {
  const dim3 grid(n_rows * a.Hq);
  if (D == 64) hipLaunchKernelGGL(attn_merge_kernel<64>, grid, dim3(64), 0, s, a);
  if (D == 128) hipLaunchKernelGGL(attn_merge_kernel<128>, grid, dim3(128), 0, s, a);
  if (D == 256) hipLaunchKernelGGL(attn_merge_kernel<256>, grid, dim3(256), 0, s, a);
}

void launch_attn_f32(const AttnF32Args &a, int n_rows, hipStream_t s) {
  hipLaunchKernelGGL(attn_f32_kernel, dim3(n_rows * a.Hq), dim3(256), 0, s, a);
}

}  // namespace sv
