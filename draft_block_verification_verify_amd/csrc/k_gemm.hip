// W_o and LM-head projections for the verify step (gfx950).
//
// Both are out[rows, N] = act[rows, K] . W[N, K]^T with a large, row-major
// weight streamed once from HBM and a small activation block (the verify
// rows).  The LM head spans the whole vocabulary (the full-vocab projection
// is what makes a one-layer predictor expensive: VESSL "Speculative Decoding
// Part 2", MTP section), so its epilogue also reduces every N tile to
// (max, sum exp, argmax) per row, ready for the vocab-wide softmax.
//
// Skinny launch (rows <= 64, HBM-bound): no LDS.  Each wavefront owns WV x 32
// weight rows and streams them straight into MFMA A-operand registers, 64
// contiguous bytes per lane per 64-wide K block; the activation fragments
// come from L2.  The K index inside a 64-block is permuted identically on
// both operands so that every lane reads contiguous memory.  The activations
// are a bf16 pair hi + lo (two bf16 MFMAs against the exact bf16 weights),
// which costs MFMA time this launch has to spare.
//
// Tiled launch (rows > 64, near the compute ridge): 256 x 256 output tiles,
// 8 wavefronts, K steps of 64 double-buffered through LDS, 32x32x16 fp16
// MFMA with fp32 accumulation.  Weight tiles are converted bf16 -> fp16 on
// their way into LDS (exact for weights in the fp16 normal range) and the
// activations arrive in fp16, so the activations keep 11 significant bits
// at no extra MFMA work.
#include "k_common.hpp"
#include "launch.hpp"

namespace sv {

// ----------------------------------------------------------------------------
// epilogue shared by both launches: acc[v][t] holds, for lane (r32, kg),
// D[n = nb[v] + 8*(j/4) + 4*kg + (j%4)][token = tb[t] + r32], j = 0..15.
// ----------------------------------------------------------------------------

template <int NV, int NT>
__device__ __forceinline__ void store_tile(const GemmArgs &g, const f32x16 (&acc)[NV][NT], const int (&nb)[NV],
                                           const int (&tb)[NT], int lane) {
  const int r32 = lane & 31, kg = lane >> 5;
  float *base = g.out;
  const bool vec = (g.N % 4) == 0;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int tok = tb[t] + r32;
    if (tok >= g.rows) continue;
    float *orow = base + int64_t(tok) * g.ldo;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n0 = nb[v] + 8 * q + 4 * kg;
        if (vec && n0 + 3 < g.N) {
          *reinterpret_cast<f32x4 *>(orow + n0) =
              f32x4{acc[v][t][4 * q], acc[v][t][4 * q + 1], acc[v][t][4 * q + 2], acc[v][t][4 * q + 3]};
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n0 + e < g.N) orow[n0 + e] = acc[v][t][4 * q + e];
        }
      }
    }
  }
}

// Per-lane (max, sumexp, argmax) over the lane's N values of token block t,
// merged with the partner lane (l ^ 32) holding the other N rows.
template <int NV, int NT>
__device__ __forceinline__ MaxSumArg lane_stats(const GemmArgs &g, const f32x16 (&acc)[NV][NT], const int (&nb)[NV],
                                                int t, int lane) {
  const int kg = lane >> 5;
  float m = -INFINITY;
  int arg = 0x7fffffff;
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int n = nb[v] + 8 * (j >> 2) + 4 * kg + (j & 3);
      const float x = acc[v][t][j];
      if (n < g.N && (x > m || (x == m && n < arg))) {
        m = x;
        arg = n;
      }
    }
  float s = 0.f;
  if (m != -INFINITY) {
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int n = nb[v] + 8 * (j >> 2) + 4 * kg + (j & 3);
        if (n < g.N) s += __expf(acc[v][t][j] - m);
      }
  }
  MaxSumArg r{m, s, arg};
  return msa_shfl_xor(r, 32);
}

// ----------------------------------------------------------------------------
// skinny launch
// ----------------------------------------------------------------------------

template <int TB, int WV, bool STATS>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(GemmArgs g) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r32 = lane & 31, kg = lane >> 5;
  constexpr int WG_N = 4 * WV * 32;
  const int n_wave = blockIdx.x * WG_N + w * WV * 32;
  const int ks = blockIdx.y * g.k_split;
  const int ke = min(g.K, ks + g.k_split);

  const uint16_t *wp[WV];
#pragma unroll
  for (int v = 0; v < WV; ++v) {
    const int n = min(n_wave + v * 32 + r32, g.N - 1);
    wp[v] = g.W + int64_t(n) * g.K + kg * 32;
  }
  const uint16_t *ap[TB];
#pragma unroll
  for (int t = 0; t < TB; ++t) {
    const int row = min(t * 32 + r32, g.rows - 1);
    ap[t] = g.act + int64_t(row) * g.K + kg * 32;
  }
  const int64_t lo_off = g.act_lo - g.act;
  f32x16 acc[WV][TB];
#pragma unroll
  for (int v = 0; v < WV; ++v)
#pragma unroll
    for (int t = 0; t < TB; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[v][t][j] = 0.f;

  uint4 wa[WV][4], wb[WV][4];
  auto load_w = [&](uint4 (&dst)[WV][4], int k) {
#pragma unroll
    for (int v = 0; v < WV; ++v)
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[v][j] = ld_nt16(wp[v] + k + 8 * j);
  };
  auto compute = [&](const uint4 (&src)[WV][4], int k) {
    uint4 bh[TB][4], bl[TB][4];
#pragma unroll
    for (int t = 0; t < TB; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bh[t][j] = reinterpret_cast<const uint4 *>(ap[t] + k)[j];
        bl[t][j] = reinterpret_cast<const uint4 *>(ap[t] + lo_off + k)[j];
      }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < WV; ++v)
#pragma unroll
        for (int t = 0; t < TB; ++t) {
          acc[v][t] = mfma32(src[v][j], bh[t][j], acc[v][t]);
          acc[v][t] = mfma32(src[v][j], bl[t][j], acc[v][t]);
        }
  };

  if (ks < ke) load_w(wa, ks);
  for (int k = ks; k < ke; k += 128) {
    if (k + 64 < ke) load_w(wb, k + 64);
    compute(wa, k);
    if (k + 64 < ke) {
      if (k + 128 < ke) load_w(wa, k + 128);
      compute(wb, k + 64);
    }
  }

  int nb[WV], tb[TB];
#pragma unroll
  for (int v = 0; v < WV; ++v) nb[v] = n_wave + v * 32;
#pragma unroll
  for (int t = 0; t < TB; ++t) tb[t] = t * 32;
  GemmArgs go = g;
  go.out = g.out + int64_t(blockIdx.y) * g.split_stride;
  store_tile<WV, TB>(go, acc, nb, tb, lane);

  if constexpr (STATS) {
    __shared__ MaxSumArg red[4][TB * 32];
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      const MaxSumArg r = lane_stats<WV, TB>(g, acc, nb, t, lane);
      if (kg == 0) red[w][t * 32 + r32] = r;
    }
    __syncthreads();
    if (tid < TB * 32 && tid < g.rows) {
      MaxSumArg r = red[0][tid];
#pragma unroll
      for (int ww = 1; ww < 4; ++ww) r = msa_merge(r, red[ww][tid]);
      const int64_t o = int64_t(tid) * g.n_tiles + blockIdx.x;
      g.t_max[o] = r.m;
      g.t_sum[o] = r.s;
      g.t_arg[o] = r.i;
    }
  }
}

// ----------------------------------------------------------------------------
// tiled launch: 256 (N) x 256 (rows) per workgroup, 8 wavefronts as 2 x 4,
// each 128 (N) x 64 (rows) = 4 x 2 MFMA blocks.
// ----------------------------------------------------------------------------

constexpr int kTBN = 256, kTBT = 256, kTKS = 64, kTROW = kTKS + 8;

template <bool STATS>
__global__ __launch_bounds__(512) void gemm_tiled_kernel(GemmArgs g) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  uint16_t *w_lds = lds;                         // [2][kTBN * kTROW]
  uint16_t *a_lds = lds + 2 * kTBN * kTROW;      // [2][kTBT * kTROW]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r32 = lane & 31, kg = lane >> 5;
  const int wn = w & 1, wt = w >> 1;
  const int n0 = blockIdx.x * kTBN;
  const int t0 = blockIdx.y * kTBT;
  const int K = g.K;

  // global -> register staging: 4 W chunks + 4 act chunks of 16 B per thread
  const uint16_t *wsrc[4];
  const uint16_t *asrc[4];
  int ldst[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = tid + 512 * j;
    const int row = c >> 3, col = c & 7;
    wsrc[j] = g.W + int64_t(min(n0 + row, g.N - 1)) * K + col * 8;
    asrc[j] = g.act + int64_t(min(t0 + row, g.rows - 1)) * K + col * 8;
    ldst[j] = row * kTROW + col * 8;
  }
  uint4 wr[4], ar[4];
  auto load = [&](int k) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      wr[j] = ld_nt16(wsrc[j] + k);
      ar[j] = *reinterpret_cast<const uint4 *>(asrc[j] + k);
    }
  };
  auto store = [&](int b) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      *reinterpret_cast<uint4 *>(w_lds + b * kTBN * kTROW + ldst[j]) = bf8_to_h8(wr[j]);
      *reinterpret_cast<uint4 *>(a_lds + b * kTBT * kTROW + ldst[j]) = ar[j];
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int v = 0; v < 4; ++v)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[v][t][j] = 0.f;

  const int nk = K / kTKS;
  load(0);
  store(0);
  __syncthreads();
  for (int s = 0; s < nk; ++s) {
    const int b = s & 1;
    if (s + 1 < nk) load((s + 1) * kTKS);
    const uint16_t *wl = w_lds + b * kTBN * kTROW + (wn * 128 + r32) * kTROW + kg * 8;
    const uint16_t *al = a_lds + b * kTBT * kTROW + (wt * 64 + r32) * kTROW + kg * 8;
#pragma unroll
    for (int kk = 0; kk < kTKS / 16; ++kk) {
      uint4 af[4], bf[2];
#pragma unroll
      for (int v = 0; v < 4; ++v) af[v] = *reinterpret_cast<const uint4 *>(wl + v * 32 * kTROW + kk * 16);
#pragma unroll
      for (int t = 0; t < 2; ++t) bf[t] = *reinterpret_cast<const uint4 *>(al + t * 32 * kTROW + kk * 16);
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int t = 0; t < 2; ++t) acc[v][t] = mfma32h(af[v], bf[t], acc[v][t]);
    }
    if (s + 1 < nk) store(b ^ 1);
    __syncthreads();
  }

  int nb[4], tb[2];
#pragma unroll
  for (int v = 0; v < 4; ++v) nb[v] = n0 + wn * 128 + v * 32;
#pragma unroll
  for (int t = 0; t < 2; ++t) tb[t] = t0 + wt * 64 + t * 32;
  store_tile<4, 2>(g, acc, nb, tb, lane);

  if constexpr (STATS) {
    MaxSumArg *red = reinterpret_cast<MaxSumArg *>(lds);   // [2][kTBT]; LDS free after the loop
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const MaxSumArg r = lane_stats<4, 2>(g, acc, nb, t, lane);
      if (kg == 0) red[wn * kTBT + wt * 64 + t * 32 + r32] = r;
    }
    __syncthreads();
    if (tid < kTBT && t0 + tid < g.rows) {
      const MaxSumArg r = msa_merge(red[tid], red[kTBT + tid]);
      const int64_t o = int64_t(t0 + tid) * g.n_tiles + blockIdx.x;
      g.t_max[o] = r.m;
      g.t_sum[o] = r.s;
      g.t_arg[o] = r.i;
    }
  }
}

constexpr size_t kTiledLds = size_t(2) * (kTBN + kTBT) * kTROW * sizeof(uint16_t);

int lm_tile_width(int rows) { return rows <= 64 ? 4 * 2 * 32 : kTBN; }

void launch_gemm_bf16(const GemmArgs &g, bool stats, int splits, hipStream_t s) {
  if (g.rows <= 64) {
    // WV = 2 for the LM head (256 N rows per workgroup), 1 for split-K W_o
    const int wv = stats ? 2 : 1;
    const dim3 grid((g.N + 4 * wv * 32 - 1) / (4 * wv * 32), splits);
#define SV_SK(TB, WV, ST) hipLaunchKernelGGL((gemm_skinny_kernel<TB, WV, ST>), grid, dim3(256), 0, s, g)
    if (g.rows <= 32) {
      if (stats) SV_SK(1, 2, true); else SV_SK(1, 1, false);
    } else {
      if (stats) SV_SK(2, 2, true); else SV_SK(2, 1, false);
    }
#undef SV_SK
    return;
  }
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(gemm_tiled_kernel<true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, int(kTiledLds));
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(gemm_tiled_kernel<false>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, int(kTiledLds));
    attr_set = true;
  }
  const dim3 grid((g.N + kTBN - 1) / kTBN, (g.rows + kTBT - 1) / kTBT);
  // split-K is not used with the tiled launch
  if (stats)
    hipLaunchKernelGGL(gemm_tiled_kernel<true>, grid, dim3(512), kTiledLds, s, g);
  else
    hipLaunchKernelGGL(gemm_tiled_kernel<false>, grid, dim3(512), kTiledLds, s, g);
}

// ----------------------------------------------------------------------------
// fp32 path: plain dot products
// ----------------------------------------------------------------------------

__global__ __launch_bounds__(64) void gemm_f32_kernel(const float *act, int rows, const float *W, int N, int K,
                                                      float *out) {
  const int n = blockIdx.x * 64 + threadIdx.x;
  const int row = blockIdx.y;
  if (n >= N) return;
  const float *a = act + int64_t(row) * K;
  const float *wr = W + int64_t(n) * K;
  float s = 0.f;
  for (int k = 0; k < K; ++k) s = fmaf(a[k], wr[k], s);
  out[int64_t(row) * N + n] = s;
}

void launch_gemm_f32(const float *act, int rows, const float *W, int N, int K, float *out, hipStream_t s) {
  hipLaunchKernelGGL(gemm_f32_kernel, dim3((N + 63) / 64, rows), dim3(64), 0, s, act, rows, W, N, K, out);
}

__global__ __launch_bounds__(256) void stats_from_logits_kernel(const float *logits, int V, int tile, float *t_max,
                                                                float *t_sum, int32_t *t_arg, int n_tiles) {
  const int c = blockIdx.x, row = blockIdx.y, tid = threadIdx.x;
  const float *lg = logits + int64_t(row) * V;
  MaxSumArg r = msa_empty();
  for (int u = c * tile + tid; u < min(V, (c + 1) * tile); u += 256) r = msa_merge(r, MaxSumArg{lg[u], 1.f, u});
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) r = msa_shfl_xor(r, o);
  __shared__ MaxSumArg red[4];
  if ((tid & 63) == 0) red[tid >> 6] = r;
  __syncthreads();
  if (tid == 0) {
    r = msa_merge(msa_merge(red[0], red[1]), msa_merge(red[2], red[3]));
    const int64_t o = int64_t(row) * n_tiles + c;
    t_max[o] = r.m;
    t_sum[o] = r.s;
    t_arg[o] = r.i;
  }
}

void launch_stats_from_logits(const float *logits, int rows, int V, int tile, float *t_max, float *t_sum,
                              int32_t *t_arg, int n_tiles, hipStream_t s) {
  hipLaunchKernelGGL(stats_from_logits_kernel, dim3(n_tiles, rows), dim3(256), 0, s, logits, V, tile, t_max, t_sum,
                     t_arg, n_tiles);
}

// ----------------------------------------------------------------------------
// final RMS norm (unit gain) over the summed split-K partials of W_o
// ----------------------------------------------------------------------------

__global__ __launch_bounds__(256) void norm_kernel(const float *part, int splits, int64_t split_stride, int hidden,
                                                   float eps, int mode, void *out, int64_t lo_off) {
  const int row = blockIdx.x, tid = threadIdx.x;
  const float *p = part + int64_t(row) * hidden;
  float ss = 0.f;
  for (int c = tid; c < hidden; c += 256) {
    float h = 0.f;
    for (int s = 0; s < splits; ++s) h += p[s * split_stride + c];
    ss = fmaf(h, h, ss);
  }
  ss = wave_sum(ss);
  __shared__ float red[4];
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  const float inv = 1.0f / sqrtf(tot / float(hidden) + eps);
  for (int c = tid; c < hidden; c += 256) {
    float h = 0.f;
    for (int s = 0; s < splits; ++s) h += p[s * split_stride + c];
    const float y = h * inv;
    const int64_t idx = int64_t(row) * hidden + c;
    if (mode == ACT_SPLIT) {
      uint16_t hi, lo;
      split_bf(y, hi, lo);
      static_cast<uint16_t *>(out)[idx] = hi;
      static_cast<uint16_t *>(out)[lo_off + idx] = lo;
    } else if (mode == ACT_F16) {
      static_cast<uint16_t *>(out)[idx] = f2h(y);
    } else {
      static_cast<float *>(out)[idx] = y;
    }
  }
}

void launch_norm(const float *part, int splits, int64_t split_stride, int rows, int hidden, float eps, int mode,
                 void *out, int64_t lo_off, hipStream_t s) {
  hipLaunchKernelGGL(norm_kernel, dim3(rows), dim3(256), 0, s, part, splits, split_stride, hidden, eps, mode, out,
                     lo_off);
}

}  // namespace sv
