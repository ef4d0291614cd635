// Vocabulary-wide reductions and acceptance for the verify step (gfx950).
//
//  drafter_partial  (max, sum exp) of every drafter-logit row, per chunk
//                   (coalesced 16-B streaming of the bf16 rows); for bf16
//                   models in one launch with the RoPE of the rows
//                   (rope_drafter).
//  row_combine      per row: max, logsumexp and greedy token of the target
//                   from the LM-head tile records; per draft row: log Z of q.
//  overlap_partial  per draft row i with parent j and per vocabulary chunk:
//                   sum_u min(p_j(u), q_i(u)) = sum_u exp(min(l_ju - lse_j,
//                   b_iu - lse_q_i)), the 1 - TV overlap (onedev.kr SpecOPD
//                   summary, "how it is used"; VESSL part 2, DSpark section).
//  accept           per tree: overlaps, prefix-survival products and their
//                   sum, and the greedy longest-matching walk with the bonus
//                   token (sionic.ai Solar Open2 page, section 1; SpecOPD
//                   summary, "premises and limits").
//  swalk / residual_partial / sample
//                   T = 1 stochastic verification of chains: the accept test
//                   per draft and the inverse-CDF draw of the bonus token.
// Every reduction runs in a fixed order, so repeated runs are bit-identical.
#include "k_common.hpp"
#include "k_rope.hpp"
#include "launch.hpp"

namespace sv {

struct MaxSum {
  float m, s;
};

__device__ __forceinline__ MaxSum ms_merge(MaxSum a, MaxSum b) {
  const float m = fmaxf(a.m, b.m);
  if (m == -INFINITY) return {m, 0.f};
  return {m, a.s * __expf(a.m - m) + b.s * __expf(b.m - m)};
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ MaxSum ms_dpp_step(MaxSum a) {
  return ms_merge(a, MaxSum{dpp_move<CTRL, ROW_MASK>(a.m, -INFINITY), dpp_move<CTRL, ROW_MASK>(a.s, 0.f)});
}

__device__ __forceinline__ MaxSum ms_block256(MaxSum r) {
  // the wavefront's (max, sum exp) on DPP moves (the sequence of wave_sum)
  r = ms_dpp_step<0xB1>(r);
  r = ms_dpp_step<0x4E>(r);
  r = ms_dpp_step<0x141>(r);
  r = ms_dpp_step<0x140>(r);
  r = ms_dpp_step<0x142, 0xA>(r);
  r = ms_dpp_step<0x143, 0xC>(r);
  r = MaxSum{__int_as_float(__builtin_amdgcn_readlane(__float_as_int(r.m), 63)),
             __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r.s), 63))};
  __shared__ MaxSum red[4];
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = r;
  __syncthreads();
  return ms_merge(ms_merge(red[0], red[1]), ms_merge(red[2], red[3]));
}

__device__ __forceinline__ float sum_block256(float v) {
  v = wave_sum(v);
  __shared__ float red[4];
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// 8 consecutive drafter logits as floats (bf16 or fp32 source)
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16 bytes with the non-temporal hint: the drafter logits and the LM head's
// fp16 probabilities are streamed by each pass once (measured under a 512 MB
// write flush before each step: the drafter-statistics pass of 224 rows x
// 248320 bf16 logits 51 -> 36 us, the overlap pass 48 -> 42 us)
__device__ __forceinline__ uint4 ld16s(const void *p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void load8(const void *base, int bf16, int64_t idx, float (&x)[8]) {
  if (bf16) {
    const uint4 u = ld16s(static_cast<const uint16_t *>(base) + idx);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int t = 0; t < 8; ++t) x[t] = __uint_as_float((t & 1) ? (w[t >> 1] & 0xFFFF0000u) : (w[t >> 1] << 16));
  } else {
    const float4 a = *reinterpret_cast<const float4 *>(static_cast<const float *>(base) + idx);
    const float4 b = *reinterpret_cast<const float4 *>(static_cast<const float *>(base) + idx + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

__device__ __forceinline__ float load1(const void *base, int bf16, int64_t idx) {
  return bf16 ? bf2f(static_cast<const uint16_t *>(base)[idx]) : static_cast<const float *>(base)[idx];
}

// ----------------------------------------------------------------------------

constexpr int kDrafterChunk = 2048;   // the host's drafter-stats chunk: vocabulary values per wavefront record

// (max, sum exp) of chunk c of drafter row t, by one wavefront: its own
// record, so that no workgroup-wide reduction or barrier sits between the
// loads and the store (a workgroup's four wavefronts take four chunks)
__device__ __forceinline__ void drafter_partial_wave(const VocabArgs &a, int c, int t) {
  const int lane = threadIdx.x & 63;
  const int lo = c * a.dchunk, hi = min(a.V, lo + a.dchunk);
  const int64_t row = int64_t(t) * a.V;
  float m = -INFINITY, s = 0.f;
  if ((a.V % 8) == 0 && a.dchunk == kDrafterChunk && a.drafter_bf16) {
    // the lane's four groups of 8 bf16 values, all loaded before use (one
    // pass over HBM) and kept packed, 4 registers per group, until each pass
    // widens them (widened on load, the pass over 224 rows x 248320 took
    // 33 -> 29 us); values past the vocabulary read as -inf
    constexpr int NG = kDrafterChunk / 512;
    uint32_t raw[NG][4];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int u = lo + lane * 8 + g * 512;
      const uint4 v = u < hi ? ld16s(static_cast<const uint16_t *>(a.drafter) + row + u)
                             : make_uint4(0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u);
      raw[g][0] = v.x;
      raw[g][1] = v.y;
      raw[g][2] = v.z;
      raw[g][3] = v.w;
    }
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        m = fmaxf(m, fmaxf(__uint_as_float(raw[g][e] << 16), __uint_as_float(raw[g][e] & 0xFFFF0000u)));
    m = wave_max(m);
    if (m != -INFINITY) {
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s += __expf(__uint_as_float(raw[g][e] << 16) - m);
          s += __expf(__uint_as_float(raw[g][e] & 0xFFFF0000u) - m);
        }
    }
  } else if ((a.V % 8) == 0 && a.dchunk == kDrafterChunk) {
    // fp32 logits: the lane's four groups of 8, all loaded before use;
    // values past the vocabulary read as -inf
    constexpr int NG = kDrafterChunk / 512;
    float x[NG][8];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int u = lo + lane * 8 + g * 512;
      if (u < hi) {
        load8(a.drafter, a.drafter_bf16, row + u, x[g]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[g][e] = -INFINITY;
      }
    }
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, x[g][e]);
    m = wave_max(m);
    if (m != -INFINITY) {
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) s += __expf(x[g][e] - m);   // exp(-inf) = 0
    }
  } else {
    for (int u = lo + lane; u < hi; u += 64) m = fmaxf(m, load1(a.drafter, a.drafter_bf16, row + u));
    m = wave_max(m);
    if (m != -INFINITY)
      for (int u = lo + lane; u < hi; u += 64) s += __expf(load1(a.drafter, a.drafter_bf16, row + u) - m);
  }
  s = wave_sum(s);
  if (lane == 0) a.dpart[int64_t(t) * a.n_dch + c] = make_float2(m, s);
}

// chunks 4 cg .. 4 cg + 3 of drafter row t, one per wavefront
__device__ __forceinline__ void drafter_partial_block(const VocabArgs &a, int cg, int t) {
  const int c = cg * 4 + int(threadIdx.x >> 6);
  if (c < a.n_dch) drafter_partial_wave(a, c, t);
}

__global__ __launch_bounds__(256) void drafter_partial_kernel(VocabArgs a) {
  drafter_partial_block(a, blockIdx.x, blockIdx.y);
}

// RoPE of the rows and the drafter statistics in one launch (independent
// work: the first is fp64 arithmetic on little data, the second a stream of
// the drafter logits, so they overlap).  Workgroups [0, n * ry) rotate row
// b / ry, pairs of block b % ry; the rest take drafter chunks.
__global__ __launch_bounds__(256) void rope_drafter_kernel(RopeArgs r, VocabArgs a) {
  const int b = blockIdx.x;
  const int nr = r.n * r.ry;
  if (b < nr) {
    rope_rows_block<uint16_t>(r.q, r.k, r.q_out, r.k_out, r.row_pos, r.Hq, r.Hkv, r.D, r.base, r.q_lo_off, r.k_lo_off,
                              b / r.ry, b % r.ry, r.ry);
  } else {
    const int d = b - nr, ncg = (a.n_dch + 3) / 4;
    drafter_partial_block(a, d % ncg, d / ncg);
  }
}

// Target (max, sum exp, argmax) of row i from its LM-head tile records:
// each thread merges its strided tiles in order, then a fixed-shape tree
// over the block; every thread gets the result.
__device__ __forceinline__ MaxSumArg row_stats_block(const VocabArgs &a, int i) {
  const int tid = threadIdx.x;
  MaxSumArg r = msa_empty();
  // the thread's tiles tid, tid + 256, ... in order, their records loaded four
  // at a time ahead of the merges
  const int64_t row0 = int64_t(i) * a.n_tiles;
  for (int c0 = tid; c0 < a.n_tiles; c0 += 4 * 256) {
    MaxSumArg v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = c0 + 256 * e;
      v[e] = c < a.n_tiles ? MaxSumArg{a.t_max[row0 + c], a.t_sum[row0 + c], a.t_arg[row0 + c]} : msa_empty();
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (c0 + 256 * e < a.n_tiles) r = msa_merge(r, v[e]);
  }
  r = msa_wave(r);
  __shared__ MaxSumArg red[4];
  __syncthreads();
  if ((tid & 63) == 0) red[tid >> 6] = r;
  __syncthreads();
  return msa_merge(msa_merge(red[0], red[1]), msa_merge(red[2], red[3]));
}

// (max, sum exp) of drafter row t from its chunk records, every thread
__device__ __forceinline__ MaxSum drafter_stats_block(const VocabArgs &a, int t) {
  MaxSum q{-INFINITY, 0.f};
  for (int c = threadIdx.x; c < a.n_dch; c += 256) {
    const float2 d = a.dpart[int64_t(t) * a.n_dch + c];
    q = ms_merge(q, MaxSum{d.x, d.y});
  }
  return ms_block256(q);
}

// ----------------------------------------------------------------------------
// Logit refinement of the tiled LM head.  That launch multiplies plain fp16
// activations (11 significant bits); on a peaked target distribution the
// rounding moves the largest probabilities by about 1e-3.  The tokens that can
// carry such an error -- first-pass probability >= 1/64, so at most 64 of
// them -- are recomputed here in fp32 from the fp16 hi + lo activation pair
// (about 22 bits), and the row's max, greedy token and logsumexp are
// corrected: with the candidates' first-pass probabilities p_c,
// lse' = lse + log((1 - sum_c p_c) + sum_c exp(l'_c - lse)).  The new logits
// replace the first-pass values in the logits buffer (or in the fp16 tile
// probabilities), so the overlap pass and the T = 1 walk and draw read them.
// Rows without a candidate (flat distributions) keep the first pass.
// ----------------------------------------------------------------------------

constexpr int kRefineMax = 64;
constexpr float kRefineLogTau = -4.1588830833596715f;   // log(1/64)

// first-pass logit of token u of row `row`
__device__ __forceinline__ float tile_logit(const VocabArgs &a, int row, int u) {
  if (a.p16) {
    const float p = h2f(a.p16[int64_t(row) * a.V + u]);
    return p > 0.f ? a.t_max[int64_t(row) * a.n_tiles + (u >> a.tile_shift)] + logf(p) : -INFINITY;
  }
  return a.logits[int64_t(row) * a.V + u];
}

// element offset of the 8-element chunk holding (r, k) (k % 8 == 0) in the
// blocked fp16 layout of the tiled LM head
__device__ __forceinline__ int64_t blocked_chunk(int64_t r, int k, int K) {
  const int R = int(r & 255), q = (k >> 3) & 3;
  return ((r >> 8) * (K >> 5) + (k >> 5)) * 8192 + R * 32 + (blk_slot(q, R) << 3);
}

__device__ __forceinline__ float dot8h(uint4 x, uint4 y) {
  const uint32_t xs[4] = {x.x, x.y, x.z, x.w}, ys[4] = {y.x, y.y, y.z, y.w};
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    s = fmaf(h2f(uint16_t(xs[e] & 0xFFFFu)), h2f(uint16_t(ys[e] & 0xFFFFu)), s);
    s = fmaf(h2f(uint16_t(xs[e] >> 16)), h2f(uint16_t(ys[e] >> 16)), s);
  }
  return s;
}

// (max, lowest index on ties) over the block; every thread gets it
__device__ __forceinline__ void max_arg_block256(float &m, int &i) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = __shfl_xor(m, o);
    const int i2 = __shfl_xor(i, o);
    if (m2 > m || (m2 == m && i2 < i)) {
      m = m2;
      i = i2;
    }
  }
  __shared__ float rm[4];
  __shared__ int ri[4];
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    rm[threadIdx.x >> 6] = m;
    ri[threadIdx.x >> 6] = i;
  }
  __syncthreads();
  m = rm[0];
  i = ri[0];
#pragma unroll
  for (int w = 1; w < 4; ++w)
    if (rm[w] > m || (rm[w] == m && ri[w] < i)) {
      m = rm[w];
      i = ri[w];
    }
}

// Refines row `row`: on return thread 0's r (max, argmax) and lse hold the
// corrected values.  Called by the whole workgroup.
__device__ void refine_row(const VocabArgs &a, int row, MaxSumArg &r, float &lse) {
  __shared__ int s_tile[kRefineMax], s_cand[kRefineMax];
  __shared__ float s_old[kRefineMax], s_new[kRefineMax];
  __shared__ int s_nt, s_nc;
  const int tid = threadIdx.x;
  const float thr = lse + kRefineLogTau;
  if (tid == 0) s_nt = s_nc = 0;
  __syncthreads();
  // candidate tiles (a token of probability >= 1/64); the best token of the
  // other tiles
  float ncm = -INFINITY;
  int nci = 0x7fffffff;
  const int64_t rt = int64_t(row) * a.n_tiles;
  for (int c = tid; c < a.n_tiles; c += 256) {
    const float m = a.t_max[rt + c];
    if (m >= thr) {
      const int k = atomicAdd(&s_nt, 1);
      if (k < kRefineMax) s_tile[k] = c;
    } else if (m > ncm || (m == ncm && a.t_arg[rt + c] < nci)) {
      ncm = m;
      nci = a.t_arg[rt + c];
    }
  }
  __syncthreads();
  const int nt = s_nt;
  if (nt == 0 || nt > kRefineMax) return;      // (workgroup-uniform) no candidate: the first pass stands
  // candidate tokens of those tiles; the others join the best non-candidate
  for (int j = 0; j < nt; ++j) {
    const int u = s_tile[j] * 256 + tid;
    if (u >= a.V) continue;
    const float l = tile_logit(a, row, u);
    if (l >= thr) {
      const int k = atomicAdd(&s_nc, 1);
      if (k < kRefineMax) s_cand[k] = u;
    } else if (l > ncm || (l == ncm && u < nci)) {
      ncm = l;
      nci = u;
    }
  }
  max_arg_block256(ncm, nci);                 // (its barriers also order s_cand / s_nc)
  const int nc = s_nc;
  if (nc > kRefineMax) return;                // (uniform) a probability total past 1 by rounding: keep the first pass
  if (tid == 0) {                             // ascending token order: a fixed summation order
    for (int j = 1; j < nc; ++j) {
      const int v = s_cand[j];
      int k = j - 1;
      while (k >= 0 && s_cand[k] > v) {
        s_cand[k + 1] = s_cand[k];
        --k;
      }
      s_cand[k + 1] = v;
    }
  }
  __syncthreads();
  // one wavefront per candidate: sum_k W[u, k] hi[k] and sum_k W[u, k] lo[k]
  const int w = tid >> 6, lane = tid & 63, K = a.rf_K;
  for (int j = w; j < nc; j += 4) {
    const int u = s_cand[j];
    float sh = 0.f, sl = 0.f;
    for (int k = lane * 8; k < K; k += 512) {
      const uint4 wv = *reinterpret_cast<const uint4 *>(a.rf_w + blocked_chunk(u, k, K));
      const uint4 hv = *reinterpret_cast<const uint4 *>(a.rf_hi + blocked_chunk(row, k, K));
      const uint4 lv = *reinterpret_cast<const uint4 *>(a.rf_lo + int64_t(row) * K + k);
      sh += dot8h(wv, hv);
      sl += dot8h(wv, lv);
    }
    sh = wave_sum(sh);
    sl = wave_sum(sl);
    if (lane == 0) {
      s_old[j] = sh;
      s_new[j] = sh + sl;
    }
  }
  __syncthreads();
  if (tid == 0) {
    float so = 0.f, sn = 0.f, bm = ncm;
    int bi = nci;
    for (int j = 0; j < nc; ++j) {
      const int u = s_cand[j];
      const float l = s_new[j];
      so += __expf(s_old[j] - lse);
      sn += __expf(l - lse);
      if (l > bm || (l == bm && u < bi)) {
        bm = l;
        bi = u;
      }
      if (a.p16)
        a.p16[int64_t(row) * a.V + u] = f2h(__expf(l - a.t_max[rt + (u >> 8)]));
      else
        a.logits[int64_t(row) * a.V + u] = l;
    }
    lse += logf(fmaxf(1.f - so, 0.f) + sn);
    r.m = bm;
    r.i = bi;
  }
}

__device__ __forceinline__ void row_combine_block(const VocabArgs &a, int i) {
  MaxSumArg r = row_stats_block(a, i);
  float lse = r.m + logf(r.s);
  if (a.rf_w) refine_row(a, i, r, lse);      // tiled LM head: thread 0's values corrected
  if (threadIdx.x == 0) {
    a.row_max[i] = r.m;
    a.row_lse[i] = lse;
    a.argmax[i] = r.i;
  }
  const int t = a.row_draft[i];
  if (t >= 0) {
    const MaxSum q = drafter_stats_block(a, t);
    if (threadIdx.x == 0) a.lse_q[t] = q.m + logf(q.s);
  }
}

__global__ __launch_bounds__(256) void row_combine_kernel(VocabArgs a) { row_combine_block(a, blockIdx.x); }

constexpr int kOverlapChunk = 8192;   // the host's overlap chunk (vocabulary values per workgroup)

// chunk c of draft row t's overlap with its parent j: A = lse of p_j, B =
// lse of q_t
__device__ __forceinline__ void overlap_block(const VocabArgs &a, int c, int t, int j, float A, float B) {
  const int tid = threadIdx.x;
  const float *lp = a.logits + int64_t(j) * a.V;
  const int64_t qrow = int64_t(t) * a.V;
  const int lo = c * a.ochunk, hi = min(a.V, lo + a.ochunk);
  float s = 0.f;
  if (a.p16) {
    // p_j(u) = p16(u) * exp(t_max - lse) within each tile of the LM head
    // (2^tile_shift tokens; the host takes this path only when V % 8 == 0)
    const uint16_t *pp = a.p16 + int64_t(j) * a.V;
    const float *tm = a.t_max + int64_t(j) * a.n_tiles;
    constexpr int NG = kOverlapChunk / 2048;   // groups of 8 per thread in a full chunk
    if (a.ochunk == kOverlapChunk && a.drafter_bf16) {
      // every group's loads issued before the arithmetic (one pass over HBM);
      // groups past the vocabulary contribute nothing
      uint4 hq[NG], hb[NG];
      float sc[NG];
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const int u = lo + tid * 8 + g * 2048;
        const bool in = u < hi;
        hq[g] = in ? ld16s(pp + u) : make_uint4(0, 0, 0, 0);
        hb[g] = in ? ld16s(static_cast<const uint16_t *>(a.drafter) + qrow + u) : make_uint4(0, 0, 0, 0);
        sc[g] = in ? tm[u >> a.tile_shift] : -INFINITY;
      }
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        if (lo + tid * 8 + g * 2048 >= hi) continue;
        const float scale = __expf(sc[g] - A);
        const uint32_t w[4] = {hq[g].x, hq[g].y, hq[g].z, hq[g].w};
        const uint32_t d[4] = {hb[g].x, hb[g].y, hb[g].z, hb[g].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = h2f(uint16_t((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu))) * scale;
          const float b = __uint_as_float((e & 1) ? (d[e >> 1] & 0xFFFF0000u) : (d[e >> 1] << 16));
          s += fminf(p, __expf(b - B));
        }
      }
    } else {
    for (int u = lo + tid * 8; u < hi; u += 256 * 8) {
      float b[8];
      load8(a.drafter, a.drafter_bf16, qrow + u, b);
      const uint4 h = *reinterpret_cast<const uint4 *>(pp + u);
      const float sc = __expf(tm[u >> a.tile_shift] - A);
      const uint32_t w[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = h2f(uint16_t((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu))) * sc;
        s += fminf(p, __expf(b[e] - B));
      }
    }
    }
  } else if ((a.V % 8) == 0) {
    constexpr int NG = kOverlapChunk / 2048;
    if (a.ochunk == kOverlapChunk) {
      // every group's loads issued before the arithmetic (same order of adds)
      float b[NG][8];
      float4 l0[NG], l1[NG];
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const int u = lo + tid * 8 + g * 2048;
        if (u < hi) {
          load8(a.drafter, a.drafter_bf16, qrow + u, b[g]);
          l0[g] = *reinterpret_cast<const float4 *>(lp + u);
          l1[g] = *reinterpret_cast<const float4 *>(lp + u + 4);
        }
      }
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        if (lo + tid * 8 + g * 2048 >= hi) continue;
        const float l[8] = {l0[g].x, l0[g].y, l0[g].z, l0[g].w, l1[g].x, l1[g].y, l1[g].z, l1[g].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) s += __expf(fminf(l[e] - A, b[g][e] - B));
      }
    } else {
      for (int u = lo + tid * 8; u < hi; u += 256 * 8) {
        float b[8];
        load8(a.drafter, a.drafter_bf16, qrow + u, b);
        const float4 l0 = *reinterpret_cast<const float4 *>(lp + u);
        const float4 l1 = *reinterpret_cast<const float4 *>(lp + u + 4);
        const float l[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) s += __expf(fminf(l[e] - A, b[e] - B));
      }
    }
  } else {
    for (int u = lo + tid; u < hi; u += 256)
      s += __expf(fminf(lp[u] - A, load1(a.drafter, a.drafter_bf16, qrow + u) - B));
  }
  s = sum_block256(s);
  if (tid == 0) a.opart[int64_t(t) * a.n_och + c] = s;
}

__global__ __launch_bounds__(256) void overlap_partial_kernel(VocabArgs a) {
  const int t = blockIdx.y;
  const int j = a.row_parent[a.draft_row[t]];
  overlap_block(a, blockIdx.x, t, j, a.row_lse[j], a.lse_q[t]);
}

// Overlaps, survival products and the greedy walk of tree r, by a whole
// workgroup of at least 64 threads (thread k < T takes the tree's row k).
__device__ __forceinline__ void accept_tree(const VocabArgs &a, int r) {
  const int lane = threadIdx.x;
  const int s0 = a.tree_start[r], T = a.tree_rows[r];
  __shared__ float ov[kMaxTreeRows];
  __shared__ int par[kMaxTreeRows], arg[kMaxTreeRows], did[kMaxTreeRows];
  if (lane < T) {
    const int i = s0 + lane;
    const int p = a.row_parent[i];
    const int d = a.row_draft[i];
    const int am = a.argmax[i], di = a.draft_ids[i];
    float o = 1.f;
    if (p >= 0) {
      // the chunk sums in chunk order; loads issued ahead of the adds (a
      // runtime-bounded loop of loads would wait on each one): all at once
      // for up to 32 chunks (vocabularies up to 262144), else eight at a time
      const float *op = a.opart + int64_t(d) * a.n_och;
      o = 0.f;
      if (a.n_och <= 32) {
        float x[32];
#pragma unroll
        for (int e = 0; e < 32; ++e) x[e] = e < a.n_och ? op[e] : 0.f;
#pragma unroll
        for (int e = 0; e < 32; ++e)
          if (e < a.n_och) o += x[e];
      } else {
        for (int c0 = 0; c0 < a.n_och; c0 += 8) {
          float x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = c0 + e < a.n_och ? op[c0 + e] : 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (c0 + e < a.n_och) o += x[e];
        }
      }
    }
    ov[lane] = o;
    par[lane] = p < 0 ? -1 : p - s0;
    arg[lane] = am;
    did[lane] = di;
    a.overlap[i] = o;
  }
  __syncthreads();
  __shared__ float surv[kMaxTreeRows];
  if (lane == 0) {
    // survival(root) = 1, survival(i) = survival(parent) * overlap(i)
    float sum = 0.f;
    for (int k = 0; k < T; ++k) {
      surv[k] = par[k] < 0 ? 1.f : surv[par[k]] * ov[k];
      if (par[k] >= 0) sum += surv[k];
      a.survival[s0 + k] = surv[k];
    }
    a.surv_sum[r] = sum;
    // greedy walk: step to the first child (row order) carrying the current
    // row's greedy token
    int cur = 0, acc = 0;
    for (;;) {
      int nxt = -1;
      for (int k = cur + 1; k < T; ++k)
        if (par[k] == cur && did[k] == arg[cur]) {
          nxt = k;
          break;
        }
      if (nxt < 0) break;
      cur = nxt;
      ++acc;
    }
    a.accept_len[r] = acc + 1;
    a.bonus[r] = arg[cur];
    a.last_row[r] = s0 + cur;
  }
}

// The overlap chunk of the small-batch launch (fp32 logits, bf16 drafter
// logits, a full chunk): its loads are issued before the row and drafter
// statistics are merged, since they do not depend on them; the sum then
// follows overlap_block's order exactly.
struct OverlapChunk {
  static constexpr int NG = kOverlapChunk / 2048;   // groups of 8 per thread
  uint4 q[NG];                                      // drafter logits, bf16 packed
  float4 l0[NG], l1[NG];                            // the parent's logits
};

__device__ __forceinline__ bool overlap_chunk_fast(const VocabArgs &a) {
  return !a.p16 && (a.V % 8) == 0 && a.ochunk == kOverlapChunk && a.drafter_bf16;
}

__device__ __forceinline__ void overlap_chunk_load(const VocabArgs &a, int c, int t, int j, OverlapChunk &k) {
  const int tid = threadIdx.x;
  const float *lp = a.logits + int64_t(j) * a.V;
  const int64_t qrow = int64_t(t) * a.V;
  const int lo = c * a.ochunk, hi = min(a.V, lo + a.ochunk);
#pragma unroll
  for (int g = 0; g < OverlapChunk::NG; ++g) {
    const int u = lo + tid * 8 + g * 2048;
    if (u < hi) {
      k.q[g] = ld16s(static_cast<const uint16_t *>(a.drafter) + qrow + u);
      k.l0[g] = *reinterpret_cast<const float4 *>(lp + u);
      k.l1[g] = *reinterpret_cast<const float4 *>(lp + u + 4);
    }
  }
}

__device__ __forceinline__ void overlap_chunk_sum(const VocabArgs &a, int c, int t, const OverlapChunk &k, float A,
                                                  float B) {
  const int tid = threadIdx.x;
  const int lo = c * a.ochunk, hi = min(a.V, lo + a.ochunk);
  float s = 0.f;
#pragma unroll
  for (int g = 0; g < OverlapChunk::NG; ++g) {
    if (lo + tid * 8 + g * 2048 >= hi) continue;
    const float l[8] = {k.l0[g].x, k.l0[g].y, k.l0[g].z, k.l0[g].w, k.l1[g].x, k.l1[g].y, k.l1[g].z, k.l1[g].w};
    const uint32_t w[4] = {k.q[g].x, k.q[g].y, k.q[g].z, k.q[g].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float b = __uint_as_float((e & 1) ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16));
      s += __expf(fminf(l[e] - A, b - B));
    }
  }
  s = sum_block256(s);
  if (tid == 0) a.opart[int64_t(t) * a.n_och + c] = s;
}

// The same for fp16 tile-relative probabilities (the p16 path of
// overlap_block with a full chunk, the same order of adds): the
// probabilities, the drafter logits and each group's tile maximum are loaded
// before the row and drafter statistics are merged.
struct OverlapChunkP16 {
  static constexpr int NG = kOverlapChunk / 2048;   // groups of 8 per thread
  uint4 p[NG], q[NG];                               // fp16 probabilities, bf16 drafter logits
  float tm[NG];                                     // the maximum of each group's tile
};

__device__ __forceinline__ bool overlap_chunk_p16_fast(const VocabArgs &a) {
  return a.p16 && (a.V % 8) == 0 && a.ochunk == kOverlapChunk && a.drafter_bf16;
}

__device__ __forceinline__ void overlap_chunk_p16_load(const VocabArgs &a, int c, int t, int j, OverlapChunkP16 &k) {
  const int tid = threadIdx.x;
  const uint16_t *pp = a.p16 + int64_t(j) * a.V;
  const float *tm = a.t_max + int64_t(j) * a.n_tiles;
  const int64_t qrow = int64_t(t) * a.V;
  const int lo = c * a.ochunk, hi = min(a.V, lo + a.ochunk);
#pragma unroll
  for (int g = 0; g < OverlapChunkP16::NG; ++g) {
    const int u = lo + tid * 8 + g * 2048;
    const bool in = u < hi;
    k.p[g] = in ? ld16s(pp + u) : make_uint4(0, 0, 0, 0);
    k.q[g] = in ? ld16s(static_cast<const uint16_t *>(a.drafter) + qrow + u) : make_uint4(0, 0, 0, 0);
    k.tm[g] = in ? tm[u >> a.tile_shift] : -INFINITY;
  }
}

__device__ __forceinline__ void overlap_chunk_p16_sum(const VocabArgs &a, int c, int t, const OverlapChunkP16 &k,
                                                      float A, float B) {
  const int tid = threadIdx.x;
  const int lo = c * a.ochunk, hi = min(a.V, lo + a.ochunk);
  float s = 0.f;
#pragma unroll
  for (int g = 0; g < OverlapChunkP16::NG; ++g) {
    if (lo + tid * 8 + g * 2048 >= hi) continue;
    const float scale = __expf(k.tm[g] - A);
    const uint32_t w[4] = {k.p[g].x, k.p[g].y, k.p[g].z, k.p[g].w};
    const uint32_t d[4] = {k.q[g].x, k.q[g].y, k.q[g].z, k.q[g].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = h2f(uint16_t((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu))) * scale;
      const float b = __uint_as_float((e & 1) ? (d[e >> 1] & 0xFFFF0000u) : (d[e >> 1] << 16));
      s += fminf(p, __expf(b - B));
    }
  }
  s = sum_block256(s);
  if (tid == 0) a.opart[int64_t(t) * a.n_och + c] = s;
}

// Small batches: the row statistics and the overlap sums in one launch.
// Workgroups [0, n) combine row b; the rest take overlap chunks, each
// merging its parent's and its drafter row's records itself with the same
// code and order as the combining workgroups (so with the same values).
//
// ACCEPT: a tree is complete when its T combine workgroups and the n_och
// overlap workgroups of each of its T - 1 draft rows are done; each counts
// itself in the tree's counter (after a device-scope release of its
// results), and the one that brings the count to T + (T - 1) n_och runs the
// tree's acceptance walk after a device-scope acquire.  No workgroup waits
// on another.  A device-scope release writes back the XCD's L2, which costs
// about a microsecond per workgroup: the host takes this form only for
// launches of at most kFusedAcceptMaxBlocks workgroups (8 rows over 151936
// tokens: 141 workgroups, 20 -> 16 us with acceptance included; 17 rows over
// 248320 tokens: 513 workgroups, 23 -> 71 us, so there the walk keeps its
// own launch).
template <bool ACCEPT>
__global__ __launch_bounds__(256) void combine_overlap_kernel(VocabArgs a) {
  const int b = blockIdx.x;
  int tree;
  if (b < a.n) {
    row_combine_block(a, b);
    tree = a.row_tree[b];
  } else {
    const int d = b - a.n, c = d % a.n_och, t = d / a.n_och;
    const int j = a.row_parent[a.draft_row[t]];
    if (overlap_chunk_fast(a)) {
      OverlapChunk k;
      overlap_chunk_load(a, c, t, j, k);
      const MaxSumArg r = row_stats_block(a, j);
      const MaxSum q = drafter_stats_block(a, t);
      overlap_chunk_sum(a, c, t, k, r.m + logf(r.s), q.m + logf(q.s));
    } else if (overlap_chunk_p16_fast(a)) {
      OverlapChunkP16 k;
      overlap_chunk_p16_load(a, c, t, j, k);
      const MaxSumArg r = row_stats_block(a, j);
      const MaxSum q = drafter_stats_block(a, t);
      overlap_chunk_p16_sum(a, c, t, k, r.m + logf(r.s), q.m + logf(q.s));
    } else {
      const MaxSumArg r = row_stats_block(a, j);
      const MaxSum q = drafter_stats_block(a, t);
      overlap_block(a, c, t, j, r.m + logf(r.s), q.m + logf(q.s));
    }
    tree = a.row_tree[a.draft_row[t]];
  }
  if constexpr (!ACCEPT) return;
  __shared__ int last;
  __syncthreads();   // every thread's stores issued and visible in the workgroup
  if (threadIdx.x == 0) {
    __threadfence();
    const int T = a.tree_rows[tree];
    const int old = atomicAdd(a.tree_done + tree, 1);
    last = old == T + (T - 1) * a.n_och - 1;
    if (last) __threadfence();
  }
  __syncthreads();
  if (last) accept_tree(a, tree);
}

// One workgroup per tree (at most 64 rows).
__global__ __launch_bounds__(64) void accept_kernel(VocabArgs a) { accept_tree(a, blockIdx.x); }

// ----------------------------------------------------------------------------
// T = 1 stochastic verification of chains.  One thread walks each chain (at
// most 64 rows): the draft d of child c of row cur is accepted when
// u_accept[c] * q_c(d) < p_cur(d).  The bonus weights of the stop row are
// max(0, p_cur - q_c) after a rejection of child c, or p_cur after a leaf.
// The draw sums them per 8192-token chunk (coalesced, fixed order), then
// selects by prefix sums: the chunk, the 32-token segment inside it and the
// token inside that, each the first with weight whose running total passes
// the remaining target (u_bonus times the total weight).  Where rounding puts
// the target past every prefix, the last entry with weight is taken.  All
// orders are fixed, so repeated runs draw the same token.
// ----------------------------------------------------------------------------

constexpr int kSampChunk = 8192;   // tokens per chunk

__device__ __forceinline__ float drafter_at(const VocabArgs &a, int draft, int u) {
  return load1(a.drafter, a.drafter_bf16, int64_t(draft) * a.V + u);
}

// target probability p_row(u): from the fp32 logits, or from the LM head's
// fp16 probabilities relative to their tile's maximum
__device__ __forceinline__ float p_at(const VocabArgs &a, int row, int u) {
  if (a.p16)
    return h2f(a.p16[int64_t(row) * a.V + u]) *
           __expf(a.t_max[int64_t(row) * a.n_tiles + (u >> a.tile_shift)] - a.row_lse[row]);
  return __expf(a.logits[int64_t(row) * a.V + u] - a.row_lse[row]);
}

__global__ __launch_bounds__(64) void swalk_kernel(VocabArgs a, SampleArgs sa) {
  const int r = blockIdx.x;
  if (threadIdx.x != 0) return;
  int cur = a.tree_start[r], acc = 0;
  int c;
  while ((c = sa.row_child[cur]) >= 0) {
    const int d = a.draft_ids[c];
    // a token outside the vocabulary has target probability 0: rejected,
    // and nothing is loaded for it
    if (d < 0 || d >= a.V) break;
    const float pd = p_at(a, cur, d);
    const int dr = a.row_draft[c];
    const float qd = __expf(drafter_at(a, dr, d) - a.lse_q[dr]);
    if (!(sa.u_accept[c] * qd < pd)) break;
    cur = c;
    ++acc;
  }
  a.accept_len[r] = acc + 1;
  a.last_row[r] = cur;
  sa.rej_child[r] = sa.row_child[cur];
}

// Bonus weights of one stop row: p_stop(u), or max(0, p_stop(u) - q_c(u))
// after the rejection of child c (rej = c; -1 after a leaf).
struct BonusRow {
  const float *lp;      // logits of the stop row
  const uint16_t *pp;   // or its fp16 tile-relative probabilities (a.p16)
  const float *tm;      // and their tile maxima
  const void *lq;       // drafter logits of the rejected child (resid only)
  float lse_p, lse_q;
  bool resid;
};

__device__ __forceinline__ BonusRow bonus_row(const VocabArgs &a, int stop, int rej) {
  BonusRow b;
  b.lp = a.logits + int64_t(stop) * a.V;
  b.pp = a.p16 ? a.p16 + int64_t(stop) * a.V : nullptr;
  b.tm = a.t_max + int64_t(stop) * a.n_tiles;
  b.lse_p = a.row_lse[stop];
  b.resid = rej >= 0;
  const int dr = b.resid ? a.row_draft[rej] : 0;
  b.lq = a.drafter_bf16 ? static_cast<const void *>(static_cast<const uint16_t *>(a.drafter) + int64_t(dr) * a.V)
                        : static_cast<const void *>(static_cast<const float *>(a.drafter) + int64_t(dr) * a.V);
  b.lse_q = b.resid ? a.lse_q[dr] : 0.f;
  return b;
}

constexpr int kSampPer = kSampChunk / 256;   // tokens per thread in a chunk

// weights of tokens base + tid + 256 j, j < kSampPer (0 past the vocabulary);
// every load is issued before the arithmetic
__device__ __forceinline__ void chunk_weights(const VocabArgs &a, const BonusRow &b, int base,
                                              float (&w)[kSampPer]) {
  float pr[kSampPer];   // p of the stop row
  if (b.pp) {
    // token u = base + thread + 256 j lies in tile u >> tile_shift
    uint16_t h[kSampPer];
#pragma unroll
    for (int j = 0; j < kSampPer; ++j) {
      const int u = base + int(threadIdx.x) + 256 * j;
      h[j] = u < a.V ? b.pp[u] : uint16_t(0);
    }
#pragma unroll
    for (int j = 0; j < kSampPer; ++j) {
      const int tile = min((base + int(threadIdx.x) + 256 * j) >> a.tile_shift, a.n_tiles - 1);
      pr[j] = h2f(h[j]) * __expf(b.tm[tile] - b.lse_p);
    }
  } else {
    float lg[kSampPer];
#pragma unroll
    for (int j = 0; j < kSampPer; ++j) {
      const int u = base + int(threadIdx.x) + 256 * j;
      lg[j] = u < a.V ? b.lp[u] : -INFINITY;
    }
#pragma unroll
    for (int j = 0; j < kSampPer; ++j) pr[j] = __expf(lg[j] - b.lse_p);
  }
  if (b.resid) {
    float lq[kSampPer];
#pragma unroll
    for (int j = 0; j < kSampPer; ++j) {
      const int u = min(base + int(threadIdx.x) + 256 * j, a.V - 1);
      lq[j] = load1(b.lq, a.drafter_bf16, u);
    }
#pragma unroll
    for (int j = 0; j < kSampPer; ++j) w[j] = fmaxf(pr[j] - __expf(lq[j] - b.lse_q), 0.f);
  } else {
#pragma unroll
    for (int j = 0; j < kSampPer; ++j) w[j] = pr[j];
  }
}

// chunk sum: thread t adds its weights in j order, then the block adds the
// thread sums in a fixed tree (sum_block256)
__device__ __forceinline__ float chunk_sum(const VocabArgs &a, const BonusRow &b, int k) {
  float w[kSampPer];
  chunk_weights(a, b, k * kSampChunk, w);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kSampPer; ++j) s += w[j];
  return sum_block256(s);
}

__global__ __launch_bounds__(256) void residual_partial_kernel(VocabArgs a, SampleArgs sa) {
  const int k = blockIdx.x, r = blockIdx.y;
  const float s = chunk_sum(a, bonus_row(a, a.last_row[r], sa.rej_child[r]), k);
  if (threadIdx.x == 0) sa.rpart[int64_t(r) * a.n_och + k] = s;
}

// inclusive prefix sum over the 64 lanes of a wave (Kogge-Stone order)
__device__ __forceinline__ float wave_incl_scan(float v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

__device__ __forceinline__ int first_lane(uint64_t m) { return __builtin_ctzll(m); }
__device__ __forceinline__ int last_lane(uint64_t m) { return 63 - __builtin_clzll(m); }

// Select among n weights w[0..n) (LDS, n <= 64 * passes) by one wave: the
// first index with positive weight whose inclusive prefix exceeds `target`,
// else the last index with positive weight, else -1.  Writes the chosen
// index and the target less the prefix before it (clamped to the index's
// weight) through lane 0.
__device__ __forceinline__ void wave_select(const float *w, int n, float target, int *sel, float *rest) {
  const int lane = threadIdx.x & 63;
  float carry = 0.f;
  int found = -1, last = -1;
  float excl = 0.f;
  for (int b = 0; b < n && found < 0; b += 64) {
    const int i = b + lane;
    const float x = i < n ? w[i] : 0.f;
    const float S = carry + wave_incl_scan(x);
    const uint64_t hit = __ballot(x > 0.f && S > target);
    const uint64_t pos = __ballot(x > 0.f);
    if (hit) {
      const int f = first_lane(hit);
      found = b + f;
      excl = __shfl(S - x, f, 64);
    } else if (pos) {
      last = b + last_lane(pos);
    }
    carry = __shfl(S, 63, 64);
  }
  if (lane == 0) {
    if (found >= 0) {
      *sel = found;
      *rest = fminf(fmaxf(target - excl, 0.f), w[found]);
    } else {
      *sel = last;
      *rest = last >= 0 ? w[last] : 0.f;
    }
  }
}

// Draw: one workgroup per tree.  With zero residual mass the weights fall
// back to p of the stop row (chunk sums then recomputed here).
__global__ __launch_bounds__(256) void sample_kernel(VocabArgs a, SampleArgs sa) {
  __shared__ float w_lds[kSampChunk];
  __shared__ float part[256];
  __shared__ float zc[1024];
  __shared__ int sh_sel, sh_tok;
  __shared__ float sh_rest, sh_rest2;
  const int r = blockIdx.x, tid = threadIdx.x;
  const int stop = a.last_row[r];
  const int rej0 = sa.rej_child[r];
  const float *rp = sa.rpart + int64_t(r) * a.n_och;
  float zl = 0.f;
  for (int k = tid; k < a.n_och; k += 256) {
    const float x = rp[k];
    zc[k] = x;
    zl += x;
  }
  float Z = sum_block256(zl);
  const int rej = Z > 0.f ? rej0 : -1;
  const BonusRow br = bonus_row(a, stop, rej);
  if (rej != rej0) {   // zero residual mass: weights p of the stop row
    for (int k = 0; k < a.n_och; ++k) {
      const float x = chunk_sum(a, br, k);
      if (tid == 0) zc[k] = x;
    }
    __syncthreads();
    zl = 0.f;
    for (int k = tid; k < a.n_och; k += 256) zl += zc[k];
    Z = sum_block256(zl);
  }
  __syncthreads();
  if (tid < 64) wave_select(zc, a.n_och, sa.u_bonus[r] * Z, &sh_sel, &sh_rest);
  __syncthreads();
  const int chunk = max(sh_sel, 0);
  const float target = sh_rest;
  const int base = chunk * kSampChunk;
  {
    float w[kSampPer];
    chunk_weights(a, br, base, w);
#pragma unroll
    for (int j = 0; j < kSampPer; ++j) w_lds[tid + 256 * j] = w[j];
  }
  __syncthreads();
  {   // token-order segments of 32
    const float4 *w4 = reinterpret_cast<const float4 *>(w_lds + tid * 32);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float4 x = w4[j];
      s += x.x;
      s += x.y;
      s += x.z;
      s += x.w;
    }
    part[tid] = s;
  }
  __syncthreads();
  if (tid < 64) wave_select(part, 256, target, &sh_sel, &sh_rest);
  __syncthreads();
  if (tid < 64) {
    const int seg = sh_sel;
    if (seg < 0) {   // no weight in the chunk (only with no mass at all)
      if (tid == 0) a.bonus[r] = min(base, a.V - 1);
      return;
    }
    wave_select(w_lds + seg * 32, 32, sh_rest, &sh_tok, &sh_rest2);
    if (tid == 0) a.bonus[r] = base + seg * 32 + max(sh_tok, 0);
  }
}

void launch_sample(const VocabArgs &a, const SampleArgs &sa, hipStream_t s) {
  hipLaunchKernelGGL(swalk_kernel, dim3(a.R), dim3(64), 0, s, a, sa);
  hipLaunchKernelGGL(residual_partial_kernel, dim3(a.n_och, a.R), dim3(256), 0, s, a, sa);
  hipLaunchKernelGGL(sample_kernel, dim3(a.R), dim3(256), 0, s, a, sa);
}

void launch_rope_drafter_bf16(const RopeArgs &r, const VocabArgs &a, hipStream_t s) {
  const int blocks = r.n * r.ry + (a.n_dch + 3) / 4 * a.n_draft;
  hipLaunchKernelGGL(rope_drafter_kernel, dim3(blocks), dim3(256), 0, s, r, a);
}

void launch_drafter_partial(const VocabArgs &a, hipStream_t s) {
  if (a.n_draft == 0) return;
  hipLaunchKernelGGL(drafter_partial_kernel, dim3((a.n_dch + 3) / 4, a.n_draft), dim3(256), 0, s, a);
}
void launch_row_combine(const VocabArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(row_combine_kernel, dim3(a.n), dim3(256), 0, s, a);
}
bool combine_overlap_accepts(const VocabArgs &a) { return a.n + a.n_och * a.n_draft <= kFusedAcceptMaxBlocks; }

void launch_combine_overlap(const VocabArgs &a, hipStream_t s) {
  if (combine_overlap_accepts(a))
    hipLaunchKernelGGL(combine_overlap_kernel<true>, dim3(a.n + a.n_och * a.n_draft), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(combine_overlap_kernel<false>, dim3(a.n + a.n_och * a.n_draft), dim3(256), 0, s, a);
}
void launch_overlap_partial(const VocabArgs &a, hipStream_t s) {
  if (a.n_draft == 0) return;
  hipLaunchKernelGGL(overlap_partial_kernel, dim3(a.n_och, a.n_draft), dim3(256), 0, s, a);
}
void launch_accept(const VocabArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(accept_kernel, dim3(a.R), dim3(64), 0, s, a);
}

}  // namespace sv
