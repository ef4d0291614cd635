// Vocabulary-wide reductions and acceptance for the verify step (gfx950).
//
//  drafter_partial  (max, sum exp) of every drafter-logit row, per chunk
//                   (coalesced 16-B streaming of the bf16 rows).
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
// Every reduction runs in a fixed order, so repeated runs are bit-identical.
#include "k_common.hpp"
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

__device__ __forceinline__ MaxSum ms_block256(MaxSum r) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    MaxSum b{__shfl_xor(r.m, o), __shfl_xor(r.s, o)};
    r = ms_merge(r, b);
  }
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
__device__ __forceinline__ void load8(const void *base, int bf16, int64_t idx, float (&x)[8]) {
  if (bf16) {
    const uint4 u = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(base) + idx);
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

__global__ __launch_bounds__(256) void drafter_partial_kernel(VocabArgs a) {
  const int c = blockIdx.x, t = blockIdx.y, tid = threadIdx.x;
  const int lo = c * a.dchunk, hi = min(a.V, lo + a.dchunk);
  const int64_t row = int64_t(t) * a.V;
  const bool vec = (a.V % 8) == 0;
  // pass 1: max; pass 2: sum exp (the chunk is re-read from L2)
  float m = -INFINITY;
  if (vec) {
    for (int u = lo + tid * 8; u < hi; u += 256 * 8) {
      float x[8];
      load8(a.drafter, a.drafter_bf16, row + u, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, x[e]);
    }
  } else {
    for (int u = lo + tid; u < hi; u += 256) m = fmaxf(m, load1(a.drafter, a.drafter_bf16, row + u));
  }
  float s = 0.f;
  if (vec) {
    for (int u = lo + tid * 8; u < hi; u += 256 * 8) {
      float x[8];
      load8(a.drafter, a.drafter_bf16, row + u, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) s += __expf(x[e] - m);
    }
  } else {
    for (int u = lo + tid; u < hi; u += 256) s += __expf(load1(a.drafter, a.drafter_bf16, row + u) - m);
  }
  if (m == -INFINITY) s = 0.f;
  const MaxSum r = ms_block256(MaxSum{m, s});
  if (tid == 0) a.dpart[int64_t(t) * a.n_dch + c] = make_float2(r.m, r.s);
}

__global__ __launch_bounds__(256) void row_combine_kernel(VocabArgs a) {
  const int i = blockIdx.x, tid = threadIdx.x;
  // target tiles of row i: each thread merges its strided tiles in order, then
  // a fixed-shape tree over the block
  MaxSumArg r = msa_empty();
  for (int c = tid; c < a.n_tiles; c += 256) {
    const int64_t o = int64_t(i) * a.n_tiles + c;
    r = msa_merge(r, MaxSumArg{a.t_max[o], a.t_sum[o], a.t_arg[o]});
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) r = msa_shfl_xor(r, o);
  __shared__ MaxSumArg red[4];
  if ((tid & 63) == 0) red[tid >> 6] = r;
  __syncthreads();
  if (tid == 0) {
    r = msa_merge(msa_merge(red[0], red[1]), msa_merge(red[2], red[3]));
    a.row_max[i] = r.m;
    a.row_lse[i] = r.m + logf(r.s);
    a.argmax[i] = r.i;
  }
  const int t = a.row_draft[i];
  if (t >= 0) {
    MaxSum q{-INFINITY, 0.f};
    for (int c = tid; c < a.n_dch; c += 256) {
      const float2 d = a.dpart[int64_t(t) * a.n_dch + c];
      q = ms_merge(q, MaxSum{d.x, d.y});
    }
    q = ms_block256(q);
    if (tid == 0) a.lse_q[t] = q.m + logf(q.s);
  }
}

__global__ __launch_bounds__(256) void overlap_partial_kernel(VocabArgs a) {
  const int c = blockIdx.x, t = blockIdx.y, tid = threadIdx.x;
  const int i = a.draft_row[t];
  const int j = a.row_parent[i];
  const float A = a.row_lse[j], B = a.lse_q[t];
  const float *lp = a.logits + int64_t(j) * a.V;
  const int64_t qrow = int64_t(t) * a.V;
  const int lo = c * a.ochunk, hi = min(a.V, lo + a.ochunk);
  float s = 0.f;
  if ((a.V % 8) == 0) {
    for (int u = lo + tid * 8; u < hi; u += 256 * 8) {
      float b[8];
      load8(a.drafter, a.drafter_bf16, qrow + u, b);
      const float4 l0 = *reinterpret_cast<const float4 *>(lp + u);
      const float4 l1 = *reinterpret_cast<const float4 *>(lp + u + 4);
      const float l[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) s += __expf(fminf(l[e] - A, b[e] - B));
    }
  } else {
    for (int u = lo + tid; u < hi; u += 256)
      s += __expf(fminf(lp[u] - A, load1(a.drafter, a.drafter_bf16, qrow + u) - B));
  }
  s = sum_block256(s);
  if (tid == 0) a.opart[int64_t(t) * a.n_och + c] = s;
}

// One wavefront per tree (at most 64 rows).
__global__ __launch_bounds__(64) void accept_kernel(VocabArgs a) {
  const int r = blockIdx.x, lane = threadIdx.x;
  const int s0 = a.tree_start[r], T = a.tree_rows[r];
  __shared__ float ov[kMaxTreeRows];
  __shared__ int par[kMaxTreeRows], arg[kMaxTreeRows], did[kMaxTreeRows];
  if (lane < T) {
    const int i = s0 + lane;
    const int p = a.row_parent[i];
    float o = 1.f;
    if (p >= 0) {
      const int t = a.row_draft[i];
      o = 0.f;
      for (int c = 0; c < a.n_och; ++c) o += a.opart[int64_t(t) * a.n_och + c];
    }
    ov[lane] = o;
    par[lane] = p < 0 ? -1 : p - s0;
    arg[lane] = a.argmax[i];
    did[lane] = a.draft_ids[i];
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

void launch_drafter_partial(const VocabArgs &a, hipStream_t s) {
  if (a.n_draft == 0) return;
  hipLaunchKernelGGL(drafter_partial_kernel, dim3(a.n_dch, a.n_draft), dim3(256), 0, s, a);
}
void launch_row_combine(const VocabArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(row_combine_kernel, dim3(a.n), dim3(256), 0, s, a);
}
void launch_overlap_partial(const VocabArgs &a, hipStream_t s) {
  if (a.n_draft == 0) return;
  hipLaunchKernelGGL(overlap_partial_kernel, dim3(a.n_och, a.n_draft), dim3(256), 0, s, a);
}
void launch_accept(const VocabArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(accept_kernel, dim3(a.R), dim3(64), 0, s, a);
}

}  // namespace sv
