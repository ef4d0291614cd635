// W_o and LM-head projections for the verify step (gfx950).
//
// Both are out[rows, N] = act[rows, K] . W[N, K]^T with a large weight
// streamed once from HBM and a small activation block (the verify rows).
// The LM head spans the whole vocabulary (the full-vocab projection is what
// makes a one-layer predictor expensive: VESSL "Speculative Decoding Part 2",
// MTP section), so its epilogue also reduces every N tile to (max, sum exp,
// argmax) per row, ready for the vocab-wide softmax.
//
// The weights are the handle's fp16 copies (converted once from bf16 at
// handle creation, exact for the weights accepted there); both operands of
// every fp16 MFMA are fp16 with fp32 accumulation.  The LM head's weights,
// and W_o's for runs of more than 64 rows, are kept in a blocked layout (the
// LDS image of one DMA stage, block after block; see launch.hpp) so that
// every DMA instruction reads 1 KB of consecutive bytes.
//
// Skinny launch (rows <= 64, HBM-bound): weight rows and the activation
// stream into a 3-stage LDS ring by direct global -> LDS loads; the
// activation is an fp16 pair hi + lo (two MFMAs per product, MFMA time this
// launch has to spare), so it keeps about 22 significant bits.
//
// Tiled launch (rows > 64, near the compute ridge): persistent, 256 x 256
// output tiles, a 4-stage DMA ring, 32x32x16 fp16 MFMA; the activation is
// plain fp16 (11 significant bits), blocked like the weights.
//
// FP8 LM head (weight format SV_WEIGHTS_FP8): e4m3 codes of weights and
// activations with power-of-two row scales, the tiled launch's structure on
// 32x32x64 e4m3 MFMAs, the scales applied in the epilogue.
#include <algorithm>
#include <type_traits>

#include "k_common.hpp"
#include "k_dma.hpp"
#include "k_fp8.hpp"
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

// fp16 exp(acc - m[t]) for the lane's values: the tile's probabilities
// relative to the tile maximum of each token (g.N % 8 == 0, so every group of
// four consecutive columns is whole and 8-byte aligned).
template <int NV, int NT>
__device__ __forceinline__ void store_tile_p16(const GemmArgs &g, const f32x16 (&acc)[NV][NT], const int (&nb)[NV],
                                               const int (&tb)[NT], const float (&m)[NT], int lane) {
  const int r32 = lane & 31, kg = lane >> 5;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int tok = tb[t] + r32;
    if (tok >= g.rows) continue;
    uint16_t *orow = g.p16 + int64_t(tok) * g.ldo;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n0 = nb[v] + 8 * q + 4 * kg;
        if (n0 >= g.N) continue;
        uint32_t h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = f2h(__expf(acc[v][t][4 * q + e] - m[t]));
        *reinterpret_cast<uint2 *>(orow + n0) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
      }
    }
  }
}

// Per-lane (max, sumexp, argmax) over the lane's N values of token block t,
// merged with the partner lane (l ^ 32) holding the other N rows.  CHECK
// masks columns n >= N (only the last tile of a launch needs it).  KEEP:
// each value is replaced by its exp(x - m), m the lane's own maximum
// (returned in *m_lane), so that the caller can rescale it instead of taking
// the exponential again; the sums are the same either way.
template <int NV, int NT, bool CHECK = true, bool KEEP = false>
__device__ __forceinline__ MaxSumArg lane_stats(const GemmArgs &g, f32x16 (&acc)[NV][NT], const int (&nb)[NV],
                                                int t, int lane, float *m_lane = nullptr) {
  const int kg = lane >> 5;
  float m = -INFINITY;
  int arg = 0x7fffffff;
  if constexpr (CHECK) {
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int n = nb[v] + 8 * (j >> 2) + 4 * kg + (j & 3);
        const float x = acc[v][t][j];
        // columns grow with (v, j): a strict > keeps the lowest index on ties
        if (n < g.N && x > m) {
          m = x;
          arg = n;
        }
      }
  } else {
    // the maximum, then the first (v, j) holding it (columns grow with
    // (v, j), so that is the lowest column); the position is a constant
    // per value and becomes a column once
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int j = 0; j < 16; ++j) m = fmaxf(m, acc[v][t][j]);
    int code = 16 * NV;
#pragma unroll
    for (int v = NV - 1; v >= 0; --v)
#pragma unroll
      for (int j = 15; j >= 0; --j) code = acc[v][t][j] == m ? 16 * v + j : code;
    if (m != -INFINITY) {
      int base = nb[0];
#pragma unroll
      for (int v = 1; v < NV; ++v) base = (code >> 4) == v ? nb[v] : base;
      const int j = code & 15;
      arg = base + 8 * (j >> 2) + 4 * kg + (j & 3);
    }
  }
  // exp(x - m) as 2^(x log2 e - m log2 e), one fused multiply-add per value
  // and the same form on every path; branch-free (a lane whose columns are
  // all masked has every x = -inf, so every exp is 0, as is its sum)
  constexpr float kLog2e = 1.4426950408889634f;
  const float mL = (m == -INFINITY ? 0.f : m) * kLog2e;
  float s = 0.f;
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int n = nb[v] + 8 * (j >> 2) + 4 * kg + (j & 3);
      const float e = __builtin_amdgcn_exp2f(fmaf(acc[v][t][j], kLog2e, -mL));
      if (!CHECK || n < g.N) s += e;
      if constexpr (KEEP) acc[v][t][j] = e;
    }
  if constexpr (KEEP) *m_lane = m;
  MaxSumArg r{m, s, arg};
  return msa_shfl_xor(r, 32);
}

__device__ __forceinline__ uint4 lds16(const uint8_t *p) { return *reinterpret_cast<const uint4 *>(p); }

// ----------------------------------------------------------------------------
// skinny launch (rows <= 64): 4 wavefronts, each WV x 32 weight rows against
// all rows (TB blocks of 32).  K steps of 64 (128 B per weight row) land in a
// 3-stage LDS ring by DMA: weights [NR rows][128 B] and the activation hi and
// lo planes [TB*32 rows][128 B], row-XOR-swizzled (16-B chunk c of row R at
// slot c ^ (R & 7)).  Two fp16 MFMAs per product (activation hi + lo).
// BLOCKED (the LM head, NR = 256 or 128): the weights come from the blocked
// layout of the tiled launch; one K step is two consecutive 16 KB blocks,
// copied to LDS as they are (NR = 128: the workgroup's 8 KB half of each).
// ----------------------------------------------------------------------------

constexpr int kSkST = 3;

template <int TB, int WV>
constexpr int skinny_stage_bytes() {
  return 4 * WV * 32 * 128 + 2 * TB * 32 * 128;
}

template <int TB, int WV, bool STATS, bool BLOCKED>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(GemmArgs g) {
  constexpr int NR = 4 * WV * 32;            // weight rows per workgroup
  constexpr int WST = NR * 128;              // weight bytes per stage
  constexpr int AST = TB * 32 * 128;         // activation bytes per plane per stage
  constexpr int SST = WST + 2 * AST;
  constexpr int WI = NR / 8 / 4;             // weight DMA instructions per wave per stage
  constexpr int AI = 2 * TB * 32 / 8 / 4;    // activation DMA instructions per wave per stage
  constexpr int PER = WI + AI;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, kg = lane >> 5;
  const int n0 = blockIdx.x * NR;
  const int ks = blockIdx.y * g.k_split;
  const int nk = (min(g.K, ks + g.k_split) - ks) / 64;
  const int Kb = g.K * 2;
  // blocked weights come in 256-row blocks of 64-byte rows; a 128-row
  // workgroup takes one contiguous half (HB bytes) of each block
  static_assert(!BLOCKED || NR == 256 || NR == 128, "blocked weight tiles of 256 or 128 rows");
  // (NR == 128: two workgroups per 256-row block, taking its halves)
  constexpr int HB = NR * 64;
  const int half = (BLOCKED && NR == 128) ? int(blockIdx.x & 1) : 0;
  const i32x4 rw = BLOCKED ? make_rsrc(g.W + int64_t(blockIdx.x / (256 / NR)) * 256 * g.K, uint32_t(256 * Kb))
                           : make_rsrc(g.W + int64_t(n0) * g.K, uint32_t(min(NR, g.N - n0)) * Kb);
  const i32x4 rah = make_rsrc(g.act, uint32_t(g.rows) * Kb);
  const i32x4 ral = make_rsrc(g.act_lo, uint32_t(g.rows) * Kb);
  const uint32_t lds0 = lds_addr(smem);
  const int c8 = lane & 7;
  int woff[WI], aoff[AI];
#pragma unroll
  for (int i = 0; i < WI; ++i) {
    const int R = (w * WI + i) * 8 + (lane >> 3);
    const int j = (w * WI + i) * 1024;   // LDS byte offset of this instruction in the stage
    woff[i] = BLOCKED ? (j < HB ? j : 16384 + j - HB) + half * HB + lane * 16 : R * Kb + ((c8 ^ (R & 7)) << 4);
  }
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int ia = w * AI + i;                        // over [0, 2 * TB * 4)
    const int R = (ia % (TB * 4)) * 8 + (lane >> 3);
    aoff[i] = R * Kb + ((c8 ^ (R & 7)) << 4);
  }
  auto issue = [&](int s) {
    const uint32_t base = lds0 + (s % kSkST) * SST;
    const int soff = (ks + s * 64) * 2;
#pragma unroll
    for (int i = 0; i < WI; ++i) dma16<kNtStream>(rw, base + (w * WI + i) * 1024, woff[i], BLOCKED ? (ks / 32 + 2 * s) * 16384 : soff);
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      const int ia = w * AI + i;
      const int plane = ia / (TB * 4);
      dma16(plane ? ral : rah, base + WST + plane * AST + (ia % (TB * 4)) * 1024, aoff[i], soff);
    }
  };

  f32x16 acc[WV][TB];
#pragma unroll
  for (int v = 0; v < WV; ++v)
#pragma unroll
    for (int t = 0; t < TB; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[v][t][j] = 0.f;

  auto compute = [&](int s) {
    const uint8_t *base = smem + (s % kSkST) * SST;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = j * 2 + kg;
      uint4 af[WV], bh[TB], bl[TB];
#pragma unroll
      for (int v = 0; v < WV; ++v) {
        const int R = w * WV * 32 + v * 32 + r32;
        // blocked: chunk q of the 128-B step is chunk q & 3 of block q >> 2
        af[v] = BLOCKED ? lds16(base + (q >> 2) * HB + R * 64 + (blk_slot(q & 3, R) << 4))
                        : lds16(base + R * 128 + ((q ^ (R & 7)) << 4));
      }
#pragma unroll
      for (int t = 0; t < TB; ++t) {
        const int R = t * 32 + r32;
        bh[t] = lds16(base + WST + R * 128 + ((q ^ (R & 7)) << 4));
        bl[t] = lds16(base + WST + AST + R * 128 + ((q ^ (R & 7)) << 4));
      }
#pragma unroll
      for (int v = 0; v < WV; ++v)
#pragma unroll
        for (int t = 0; t < TB; ++t) {
          acc[v][t] = mfma32h(af[v], bh[t], acc[v][t]);
          acc[v][t] = mfma32h(af[v], bl[t], acc[v][t]);
        }
    }
  };

#pragma unroll
  for (int p = 0; p < kSkST - 1; ++p)
    if (p < nk) issue(p);
  for (int s = 0; s < nk; ++s) {
    // stage s landed (this wave's part, then everyone's); stage s-1's buffer is free
    if (s + 1 < nk) wait_and_barrier<PER>(); else wait_and_barrier<0>();
    if (s + kSkST - 1 < nk) issue(s + kSkST - 1);
    compute(s);
  }

  int nb[WV], tb[TB];
#pragma unroll
  for (int v = 0; v < WV; ++v) nb[v] = n0 + w * WV * 32 + v * 32;
#pragma unroll
  for (int t = 0; t < TB; ++t) tb[t] = t * 32;
  GemmArgs go = g;
  go.out = g.out + int64_t(blockIdx.y) * g.split_stride;
  if (!STATS || !g.p16) store_tile<WV, TB>(go, acc, nb, tb, lane);

  if constexpr (STATS) {
    __syncthreads();
    MaxSumArg *red = reinterpret_cast<MaxSumArg *>(smem);   // [4][TB * 32]
    // the statistics leave exp(x - m) in the accumulators, m the lane's
    // maximum (the fp16 probabilities below rescale them)
    float ml[TB];
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      const MaxSumArg r = lane_stats<WV, TB, true, true>(g, acc, nb, t, lane, &ml[t]);
      if (kg == 0) red[w * TB * 32 + t * 32 + r32] = r;
    }
    __syncthreads();
    if (tid < TB * 32 && tid < g.rows) {
      MaxSumArg r = red[tid];
#pragma unroll
      for (int ww = 1; ww < 4; ++ww) r = msa_merge(r, red[ww * TB * 32 + tid]);
      const int64_t o = int64_t(tid) * g.n_tiles + blockIdx.x;
      g.t_max[o] = r.m;
      g.t_sum[o] = r.s;
      g.t_arg[o] = r.i;
    }
    if (g.p16) {
        // fp16 probabilities relative to the tile maximum M of each token
        // (the value the records above hold), exp(x - m) exp(m - M), in
        // place of fp32 logits when no logits are asked for: half the bytes
        // written while the weights stream in (17 rows over 248320 x 5120
        // weights: writing half of the fp32 logits saved 23 us of 433).
        // Staged through the ring after the records (chunk cc of token row
        // rl at slot cc ^ (rl & (CPR - 1))), then stored as one run of NR
        // values per row; g.N % 8 == 0 here.
        constexpr int CPR = NR / 8;   // 16-byte chunks per row
        static_assert(4096 + TB * 32 * NR * 2 <= kSkST * SST, "the fp16 tile fits the ring");
        uint8_t *stg = smem + 4096;
        float sc[TB];
#pragma unroll
        for (int t = 0; t < TB; ++t) {
          const int rl = t * 32 + r32;
          float M = red[rl].m;
#pragma unroll
          for (int ww = 1; ww < 4; ++ww) M = fmaxf(M, red[ww * TB * 32 + rl].m);
          sc[t] = ml[t] == -INFINITY ? 0.f : __expf(ml[t] - M);
        }
#pragma unroll
        for (int t = 0; t < TB; ++t) {
          const int rl = t * 32 + r32;
#pragma unroll
          for (int v = 0; v < WV; ++v)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int cc = (w * WV + v) * 4 + q;
              uint32_t hh[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) hh[e] = f2h(acc[v][t][4 * q + e] * sc[t]);
              *reinterpret_cast<uint2 *>(stg + rl * (NR * 2) + ((cc ^ (rl & (CPR - 1))) << 4) + kg * 8) =
                  make_uint2(hh[0] | (hh[1] << 16), hh[2] | (hh[3] << 16));
            }
        }
        __syncthreads();
        const int live = min(TB * 32, g.rows);
        for (int i = tid; i < live * CPR; i += 256) {
          const int rl = i / CPR, c = i % CPR, col = n0 + c * 8;
          if (col < g.N)
            *reinterpret_cast<uint4 *>(g.p16 + int64_t(rl) * g.ldo + col) =
                *reinterpret_cast<const uint4 *>(stg + rl * (NR * 2) + ((c ^ (rl & (CPR - 1))) << 4));
        }
    }
  }
}

// ----------------------------------------------------------------------------
// tiled launch (rows > 64), persistent: each workgroup walks output tiles of
// 256 (N) x 256 (rows).  8 wavefronts as 2 x 4, each 128 (N) x 64 (rows) =
// 4 x 2 fp16 32x32x16 MFMA blocks; wave (wn, wt) takes the 32-row blocks wt
// and wt + 4, so the 64 padding rows of a 192-row tile (448 rows = 256 +
// 192) are one block of each of four waves on four different SIMDs, which
// skip its fragment reads and MFMAs (a K loop chosen per tile).  K steps of 32 (64 B per row) land in a
// 4-stage LDS ring by DMA (weights 256 rows, then activations 256 rows; 16-B
// chunk c of row R at slot blk_slot(c, R), so that any 16 consecutive rows
// of one chunk fall in 16 distinct bank groups), three steps ahead of the
// MFMAs.  BLOCKED (the LM head): both operands are stored in that same stage
// image, block after block, so each DMA instruction reads 1 KB of consecutive
// bytes; row-strided 64-byte pieces stream markedly slower from HBM and L2
// together.  When a tile's K loop ends, the epilogue (per-row max / sumexp /
// argmax of the tile, logit stores) is issued and the first stages of the
// workgroup's next tile follow at once, so the stores drain while those
// loads are in flight.  Tile order: tiles i and i+8 share the weight
// tile (with two row tiles) and are taken at the same time by workgroups on
// the same XCD, so one of the two weight reads hits that XCD's L2.
// ----------------------------------------------------------------------------

constexpr int kTBN = 256, kTBT = 256, kTST = 4, kTSST = (kTBN + kTBT) * 64;
constexpr size_t kTiledLds = size_t(kTST) * kTSST;
// LO (W_o above 64 rows): the activation is an fp16 pair hi + lo, both
// planes blocked, two MFMAs per product; a stage holds the weights and both
// planes (48 KB), in a 3-stage ring.
constexpr int kTSTLo = 3, kTSSTLo = (kTBN + 2 * kTBT) * 64;
constexpr size_t kTiledLdsLo = size_t(kTSTLo) * kTSSTLo;

template <bool STATS, bool BLOCKED, bool LO = false>
__global__ __launch_bounds__(512) void gemm_tiled_kernel(GemmArgs g) {
  static_assert(!LO || (BLOCKED && !STATS), "the hi + lo activation pair is for the blocked W_o launch");
  // PP (the LM head): waves 4-7 run half a K step behind waves 0-3 (one
  // barrier later, the same code), so one group's fragment reads overlap the
  // other group's MFMAs on each SIMD instead of every wave reading, then
  // every wave multiplying.  The lagging group waits for its share of one
  // stage more than the leading group before each barrier, and each group
  // drains its fragment reads before its mid-step barrier, so every read
  // follows every wave's copy of that stage and every refill follows every
  // wave's reads of the slot (tests/test_lm_head_protocol.py checks a model
  // of all waves' barrier sequences for 3-5 stages and 1-17 steps).  Same-box A/B, 256 rows over
  // 248320 x 5120 weights: 707 -> 671 us; 448 rows over 151936 x 4096:
  // 671 -> 641 us.
  constexpr bool PP = STATS;
  // DMA instructions per wave per stage: 2 weight + 2 activation (+ 2 lo)
  constexpr int PER = LO ? 6 : 4;
  constexpr int ST = LO ? kTSTLo : kTST;        // ring stages
  constexpr int SST = LO ? kTSSTLo : kTSST;     // bytes per stage
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, kg = lane >> 5;
  const int wn = w & 1, wt = w >> 1;
  // wave-uniform (a scalar value), so that the barriers it selects sit
  // under scalar branches
  const bool lag = __builtin_amdgcn_readfirstlane(w) >= 4;
  const int n_ttiles = (g.rows + kTBT - 1) / kTBT;
  const int n_ntiles = (g.N + kTBN - 1) / kTBN;
  const int n_tiles_all = ((n_ntiles + 7) / 8) * 8 * n_ttiles;
  const int ks = blockIdx.y * g.k_split;
  const int nk = (min(g.K, ks + g.k_split) - ks) / 32;
  const int Kb = g.K * 2;
  const uint32_t lds0 = lds_addr(smem);
  const int c4 = lane & 3;
  int off[2];     // 2 instructions of 16 rows: rows w*32 + 16 i + lane/4 (weights and activations alike)
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int R = w * 32 + i * 16 + (lane >> 2);
    off[i] = BLOCKED ? (w * 32 + i * 16) * 64 + lane * 16 : R * Kb + (blk_slot(c4, R) << 4);
  }
  // tile i -> (weight tile, row tile); i and i+8 share the weight tile
  auto tile_of = [&](int i, int &n_tile, int &t_tile) {
    const int grp = i / (8 * n_ttiles), rem = i % (8 * n_ttiles);
    n_tile = grp * 8 + rem % 8;
    t_tile = rem / 8;
  };
  struct Src {
    i32x4 rw, ra, rl;
  };
  auto src_of = [&](int n_tile, int t_tile) {
    const int n0 = n_tile * kTBN, t0 = t_tile * kTBT;
    Src r;
    if constexpr (BLOCKED) {
      // one column of blocks per 256-row tile; padding rows hold zeros (W)
      // or values whose outputs are dropped (act)
      const int64_t tb = int64_t(g.K) * 256;
      r.rw = make_rsrc(g.W + int64_t(n_tile) * tb, uint32_t(tb * 2));
      r.ra = make_rsrc(g.act + int64_t(t_tile) * tb, uint32_t(tb * 2));
      r.rl = LO ? make_rsrc(g.act_lo + int64_t(t_tile) * tb, uint32_t(tb * 2)) : r.ra;
    } else {
      r.rw = make_rsrc(g.W + int64_t(n0) * g.K, uint32_t(min(kTBN, g.N - n0)) * Kb);
      r.ra = make_rsrc(g.act + int64_t(t0) * g.K, uint32_t(min(kTBT, g.rows - t0)) * Kb);
      r.rl = r.ra;
    }
    return r;
  };
  auto issue = [&](const Src &sr, int s) {
    const uint32_t base = lds0 + (s % ST) * SST;
    const int soff = BLOCKED ? (ks / 32 + s) * 16384 : (ks + s * 32) * 2;
    // weights: the non-temporal hint when no other row tile reads them again
    if (n_ttiles == 1) {
#pragma unroll
      for (int i = 0; i < 2; ++i) dma16<kNtStream>(sr.rw, base + (w * 32 + i * 16) * 64, off[i], soff);
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) dma16(sr.rw, base + (w * 32 + i * 16) * 64, off[i], soff);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16(sr.ra, base + kTBN * 64 + (w * 32 + i * 16) * 64, off[i], soff);
    if constexpr (LO) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        dma16(sr.rl, base + (kTBN + kTBT) * 64 + (w * 32 + i * 16) * 64, off[i], soff);
    }
  };

  int tile = blockIdx.x;
  // skip tiles past the weight rows (grid rounding)
  auto valid = [&](int i) {
    if (i >= n_tiles_all) return false;
    int a, b;
    tile_of(i, a, b);
    return a < n_ntiles;
  };
  while (tile < n_tiles_all && !valid(tile)) tile += gridDim.x;
  if (tile >= n_tiles_all) return;      // whole workgroup, before any barrier
  int n_tile, t_tile;
  tile_of(tile, n_tile, t_tile);
  Src cur = src_of(n_tile, t_tile);
#pragma unroll
  for (int p = 0; p < ST - 1; ++p)
    if (p < nk) issue(cur, p);

  for (;;) {
    f32x16 acc[4][2];
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[v][t][j] = 0.f;

    if (PP && lag) {
      // half a step behind: this barrier meets the leading group's first
      // one, after which it reads stage 0, so this group's share of stage 0
      // must have landed
      const int younger0 = min(ST - 2, nk - 1);
      if (younger0 >= 2)
        wait_and_barrier<2 * PER>();
      else if (younger0 == 1)
        wait_and_barrier<PER>();
      else
        wait_and_barrier<0>();
    }
    // SK: this wave's second row block (rows wt * 32 + 128 ... + 31 of the
    // tile) is all padding, so its fragment reads and MFMAs are skipped
    auto kloop = [&](auto sk_tag) __attribute__((always_inline)) {
    constexpr bool SK = decltype(sk_tag)::value;
    for (int s = 0; s < nk; ++s) {
      // the lagging group waits for its share of stage s + 1 as well: the
      // leading group reads that stage after the next barrier
      const int younger = PP && lag ? max(0, min(ST - 3, nk - 2 - s)) : min(ST - 2, nk - 1 - s);
      if (younger >= 2)
        wait_and_barrier<2 * PER>();
      else if (younger == 1)
        wait_and_barrier<PER>();
      else
        wait_and_barrier<0>();
      if (s + ST - 1 < nk) issue(cur, s + ST - 1);
      const uint8_t *base = smem + (s % ST) * SST;
      uint4 af[2][4], bf[2][2], bl[2][2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int q = j * 2 + kg;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int R = wn * 128 + v * 32 + r32;
          af[j][v] = lds16(base + R * 64 + (blk_slot(q, R) << 4));
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          if (SK && t == 1) continue;
          const int R = wt * 32 + t * 128 + r32;
          bf[j][t] = lds16(base + kTBN * 64 + R * 64 + (blk_slot(q, R) << 4));
          if constexpr (LO) bl[j][t] = lds16(base + (kTBN + kTBT) * 64 + R * 64 + (blk_slot(q, R) << 4));
        }
      }
      if constexpr (PP) {
        // this group's reads are done (so the slot may be refilled after the
        // other group's next barrier); its MFMAs now run while the other
        // group reads
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            if (SK && t == 1) continue;
            acc[v][t] = mfma32h(af[j][v], bf[j][t], acc[v][t]);
            if constexpr (LO) acc[v][t] = mfma32h(af[j][v], bl[j][t], acc[v][t]);
          }
    }
    };
    if (t_tile * kTBT + (wt + 4) * 32 >= g.rows)
      kloop(std::true_type{});
    else
      kloop(std::false_type{});
    if (PP && !lag) asm volatile("s_barrier" ::: "memory");   // the lagging group's first barrier

    // epilogue of this tile (vector-memory waits count stores too, so the
    // next tile's loads are issued only after the stores)
    asm volatile("s_barrier" ::: "memory");   // every wave is done reading the ring
    const int n0 = n_tile * kTBN, t0 = t_tile * kTBT;
    int nb[4], tb[2];
#pragma unroll
    for (int v = 0; v < 4; ++v) nb[v] = n0 + wn * 128 + v * 32;
#pragma unroll
    for (int t = 0; t < 2; ++t) tb[t] = t0 + wt * 32 + t * 128;
    GemmArgs go = g;
    go.out = g.out + int64_t(blockIdx.y) * g.split_stride;
    if constexpr (STATS) {
      // (max, sumexp, argmax) per row over this wave's 128 N, then across
      // the two N halves through a small static LDS array
      __shared__ MaxSumArg red[2][kTBT];
      if (n0 + kTBN > g.N) {
        // last tile: columns past N (zero weights) must not take part
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int j = 0; j < 16; ++j)
              if (nb[v] + 8 * (j >> 2) + 4 * kg + (j & 3) >= g.N) acc[v][t][j] = -INFINITY;
      }
      // fp32 logits (when asked for) leave first: the statistics below
      // replace each accumulator by exp(x - the lane's maximum), which the
      // fp16 probabilities rescale
      if (!g.p16) store_tile<4, 2>(go, acc, nb, tb, lane);
      float ml[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const MaxSumArg r = lane_stats<4, 2, false, true>(g, acc, nb, t, lane, &ml[t]);
        if (kg == 0) red[wn][wt * 32 + t * 128 + r32] = r;
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (tid < kTBT && t0 + tid < g.rows) {
        const MaxSumArg r = msa_merge(red[0][tid], red[1][tid]);
        const int64_t o = int64_t(t0 + tid) * g.n_tiles + n_tile;
        g.t_max[o] = r.m;
        g.t_sum[o] = r.s;
        g.t_arg[o] = r.i;
      }
      if (g.p16) {
        // exp(x - M), M the tile maximum of the token (the value the merge
        // above writes to t_max), as exp(x - m) exp(m - M) with m the lane's
        // maximum (a lane whose columns are all past N stores none of them)
        float sc[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int row = wt * 32 + t * 128 + r32;
          const float M = fmaxf(red[0][row].m, red[1][row].m);
          sc[t] = ml[t] == -INFINITY ? 0.f : __expf(ml[t] - M);
        }
        // The tile's fp16 probabilities go through the idle ring (256 rows x
        // 512 B = its 128 KB): each lane writes its 8-byte pieces, 16-byte
        // chunk c of row r at slot c ^ (r & 31) so that a store instruction's
        // 32 rows take distinct banks, then 32 consecutive threads store
        // each row as 16-byte pieces of one 512-byte run (row-strided 8-byte
        // stores straight from the accumulators took about 17 us longer per
        // 256 x 248320 launch, 13 us per 448 x 151936).
        static_assert(kTST * kTSST == kTBT * kTBN * 2, "the fp16 tile fills the ring");
        // the lane's chunk c = 16 wn + 4 v + q of row rl (rl & 31 = r32) sits
        // at slot (16 wn ^ r32) ^ (4 v + q); xs is kept opaque so that the
        // sixteen slot addresses are formed here rather than hoisted out of
        // the tile loop (and spilled)
        int xs = (16 * wn) ^ r32;
        asm volatile("" : "+v"(xs));
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          uint8_t *rowp = smem + (wt * 32 + t * 128 + r32) * 512 + kg * 8;
#pragma unroll
          for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              uint32_t hh[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) hh[e] = f2h(acc[v][t][4 * q + e] * sc[t]);
              *reinterpret_cast<uint2 *>(rowp + ((xs ^ (4 * v + q)) << 4)) =
                  make_uint2(hh[0] | (hh[1] << 16), hh[2] | (hh[3] << 16));
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll 4
        for (int i = tid; i < kTBT * 32; i += 512) {
          const int rl = i >> 5, c = i & 31;
          const int tok = t0 + rl, col = n0 + c * 8;
          if (tok < g.rows && col < g.N)
            *reinterpret_cast<uint4 *>(g.p16 + int64_t(tok) * g.ldo + col) =
                *reinterpret_cast<const uint4 *>(smem + rl * 512 + ((c ^ (rl & 31)) << 4));
        }
      }
    } else {
      store_tile<4, 2>(go, acc, nb, tb, lane);
    }

    // the staged probabilities are read before the next tile's copies refill the ring
    if constexpr (STATS) {
      if (g.p16) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    int next = tile + gridDim.x;
    while (next < n_tiles_all && !valid(next)) next += gridDim.x;
    const bool more = next < n_tiles_all;
    int nn_tile = 0, nt_tile = 0;
    Src nsrc = cur;
    if (more) {
      tile_of(next, nn_tile, nt_tile);
      nsrc = src_of(nn_tile, nt_tile);
#pragma unroll
      for (int p = 0; p < ST - 1; ++p)
        if (p < nk) issue(nsrc, p);
    }
    if (!more) break;
    tile = next;
    n_tile = nn_tile;
    t_tile = nt_tile;
    cur = nsrc;
  }
}


// ----------------------------------------------------------------------------
// FP8 LM head: the tiled launch's structure (persistent 256 x 256 tiles, 8
// waves of 128 x 64, 4-stage DMA ring of 32 KB) on e4m3 operands in the
// blocked layout, K steps of 64 (64 bytes per row): per step one
// 32x32x64 e4m3 MFMA per 32 x 32 block, its operands 32 bytes of the lane's
// row (the two lane halves take the two halves of the step).  The epilogue
// multiplies by the row scales, then writes the tile statistics and logits.
// ----------------------------------------------------------------------------

typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ i32x8 cat8(uint4 a, uint4 b) {
  return i32x8{int(a.x), int(a.y), int(a.z), int(a.w), int(b.x), int(b.y), int(b.z), int(b.w)};
}

// D += A . B^T on e4m3 operands (format 0), unit block scales (E8M0 127 = 2^0)
__device__ __forceinline__ f32x16 mfma32_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

template <bool SPARSE>
__global__ __launch_bounds__(512) void gemm_fp8_kernel(GemmArgs g) {
  constexpr bool STATS = true;
  constexpr int PER = 4;     // DMA instructions per wave per stage (2 weight + 2 activation)
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // w wave-uniform (a scalar value), so that wave-indexed choices are scalar branches
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, kg = lane >> 5;
  const int wn = w & 1, wt = w >> 1;
  // the ping-pong K loop for full tiles only: with most waves idle on
  // padding rows (SPARSE), its second barrier per step costs more than it
  // overlaps (8 rows: 164 -> 332 us)
  constexpr bool PP = !SPARSE;
  const bool lag = PP && w >= 4;   // the lagging group of the ping-pong loop
  // the wave's two 32-row blocks: 2 wt and 2 wt + 1 with few rows (SPARSE:
  // waves whose blocks are all padding idle), else wt and wt + 4, as in the
  // fp16 tiled kernel (the padding blocks of a 192-row tile then fall to one
  // wave per SIMD)
  auto rowblk = [&](int t) { return SPARSE ? 2 * wt + t : wt + 4 * t; };
  const int n_ttiles = (g.rows + kTBT - 1) / kTBT;
  const int n_ntiles = (g.N + kTBN - 1) / kTBN;
  const int n_tiles_all = ((n_ntiles + 7) / 8) * 8 * n_ttiles;
  const int nk = g.K / 64;   // K steps of 64 e4m3 values (64 bytes per row)
  const int Kb = g.K * 2;
  const uint32_t lds0 = lds_addr(smem);
  const int c4 = lane & 3;
  int off[2];     // 2 instructions of 16 rows: rows w*32 + 16 i + lane/4 (weights and activations alike)
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int R = w * 32 + i * 16 + (lane >> 2);
    off[i] = (w * 32 + i * 16) * 64 + lane * 16;
    (void)R;
  }
  // tile i -> (weight tile, row tile); i and i+8 share the weight tile
  auto tile_of = [&](int i, int &n_tile, int &t_tile) {
    const int grp = i / (8 * n_ttiles), rem = i % (8 * n_ttiles);
    n_tile = grp * 8 + rem % 8;
    t_tile = rem / 8;
  };
  struct Src {
    i32x4 rw, ra;
    int ao[2];   // activation DMA offsets: rows past the tile's valid rows point out of range (read 0, no traffic)
  };
  auto src_of = [&](int n_tile, int t_tile) {
    const int n0 = n_tile * kTBN, t0 = t_tile * kTBT;
    Src r;
    // one column of blocks per 256-row tile: 256 * K bytes
    const int64_t tb = int64_t(g.K) * 256;
    r.rw = make_rsrc(g.W8 + int64_t(n_tile) * tb, uint32_t(tb));
    r.ra = make_rsrc(g.act8 + int64_t(t_tile) * tb, uint32_t(tb));
    (void)n0;
    const int live = SPARSE ? min(kTBT, g.rows - t0) : kTBT;
#pragma unroll
    for (int i = 0; i < 2; ++i) r.ao[i] = (w * 32 + i * 16 + (lane >> 2) < live) ? off[i] : 0x40000000;
    return r;
  };
  auto issue = [&](const Src &sr, int s) {
    const uint32_t base = lds0 + (s % kTST) * kTSST;
    const int soff = s * 16384;
    // weights: the non-temporal hint when no other row tile reads them again
    if (n_ttiles == 1) {
#pragma unroll
      for (int i = 0; i < 2; ++i) dma16<kNtStream>(sr.rw, base + (w * 32 + i * 16) * 64, off[i], soff);
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) dma16(sr.rw, base + (w * 32 + i * 16) * 64, off[i], soff);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16(sr.ra, base + kTBN * 64 + (w * 32 + i * 16) * 64, sr.ao[i], soff);
  };

  int tile = blockIdx.x;
  // skip tiles past the weight rows (grid rounding)
  auto valid = [&](int i) {
    if (i >= n_tiles_all) return false;
    int a, b;
    tile_of(i, a, b);
    return a < n_ntiles;
  };
  while (tile < n_tiles_all && !valid(tile)) tile += gridDim.x;
  if (tile >= n_tiles_all) return;      // whole workgroup, before any barrier
  int n_tile, t_tile;
  tile_of(tile, n_tile, t_tile);
  Src cur = src_of(n_tile, t_tile);
#pragma unroll
  for (int p = 0; p < kTST - 1; ++p)
    if (p < nk) issue(cur, p);

  for (;;) {
    // 32-row blocks of this wave that hold rows of the batch
    const int live_rows = g.rows - t_tile * kTBT;
    const bool live_t0 = !SPARSE || wt * 64 < live_rows, live_t1 = !SPARSE || wt * 64 + 32 < live_rows;
    f32x16 acc[4][2];
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[v][t][j] = 0.f;

    // the ping-pong K loop of the fp16 LM head (gemm_tiled_kernel, PP):
    // waves 4-7 one barrier behind waves 0-3, the same barrier sequence
    if (lag) {
      const int younger0 = min(kTST - 2, nk - 1);
      if (younger0 >= 2)
        wait_and_barrier<2 * PER>();
      else if (younger0 == 1)
        wait_and_barrier<PER>();
      else
        wait_and_barrier<0>();
    }
    // SK (full tiles only): this wave's second row block is all padding, so
    // its fragment reads and MFMAs are skipped
    auto kloop = [&](auto sk_tag) {
    constexpr bool SK = decltype(sk_tag)::value;
    const bool live1 = SPARSE ? live_t1 : !SK;
    for (int s = 0; s < nk; ++s) {
      const int younger = lag ? max(0, min(kTST - 3, nk - 2 - s)) : min(kTST - 2, nk - 1 - s);
      if (younger >= 2)
        wait_and_barrier<2 * PER>();
      else if (younger == 1)
        wait_and_barrier<PER>();
      else
        wait_and_barrier<0>();
      if (s + kTST - 1 < nk) issue(cur, s + kTST - 1);
      const uint8_t *base = smem + (s % kTST) * kTSST;
      // 32 bytes of the lane's row per operand: chunks 2 kg and 2 kg + 1
      i32x8 af[4], bf[2];
      if (live_t0) {   // else: this wave's 64 rows are all padding (copies and barriers only)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int R = wn * 128 + v * 32 + r32, sw = blk_slot(0, R);
          af[v] = cat8(lds16(base + R * 64 + (((2 * kg) ^ sw) << 4)), lds16(base + R * 64 + (((2 * kg + 1) ^ sw) << 4)));
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          if (SK && t == 1) continue;
          const int R = rowblk(t) * 32 + r32, sw = blk_slot(0, R);
          bf[t] = cat8(lds16(base + kTBN * 64 + R * 64 + (((2 * kg) ^ sw) << 4)),
                       lds16(base + kTBN * 64 + R * 64 + (((2 * kg + 1) ^ sw) << 4)));
        }
      }
      if constexpr (PP) {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
      }
      if (!live_t0) continue;
      if (live1) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int t = 0; t < 2; ++t) acc[v][t] = mfma32_fp8(af[v], bf[t], acc[v][t]);
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[v][0] = mfma32_fp8(af[v], bf[0], acc[v][0]);
      }
    }
    };
    if constexpr (SPARSE)
      kloop(std::false_type{});
    else if (t_tile * kTBT + (wt + 4) * 32 >= g.rows)
      kloop(std::true_type{});
    else
      kloop(std::false_type{});

    if (PP && !lag) asm volatile("s_barrier" ::: "memory");   // the lagging group's first barrier

    // epilogue of this tile (vector-memory waits count stores too, so the
    // next tile's loads are issued only after the stores)
    asm volatile("s_barrier" ::: "memory");   // every wave is done reading the ring
    const int n0 = n_tile * kTBN, t0 = t_tile * kTBT;
    int nb[4], tb[2];
#pragma unroll
    for (int v = 0; v < 4; ++v) nb[v] = n0 + wn * 128 + v * 32;
#pragma unroll
    for (int t = 0; t < 2; ++t) tb[t] = t0 + rowblk(t) * 32;
    GemmArgs go = g;
    // scales: logit = a_t s_n * (code products); padding rows have scale 1
    {
      const float at0 = g.a_scale[min(tb[0] + r32, g.rows - 1)], at1 = g.a_scale[min(tb[1] + r32, g.rows - 1)];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float4 *ws = reinterpret_cast<const float4 *>(g.w_scale + nb[v] + 4 * kg);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 w4 = ws[2 * q];   // columns nb[v] + 8 q + 4 kg + 0..3
          const float wv[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[v][0][4 * q + e] *= at0 * wv[e];
            acc[v][1][4 * q + e] *= at1 * wv[e];
          }
        }
      }
    }
    if constexpr (STATS) {
      // the fp16 tiled kernel's epilogue, line for line: (max, sumexp,
      // argmax) per row over this wave's 128 N, then across the two N halves
      // through a small static LDS array, then fp32 logits or staged fp16
      // probabilities.  (Kept inline in both kernels: as one shared
      // function the compiler held more kernel arguments in scalar registers
      // across the K loop and spilled them there.)
      __shared__ MaxSumArg red[2][kTBT];
      if (n0 + kTBN > g.N) {
        // last tile: columns past N (zero weights) must not take part
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int j = 0; j < 16; ++j)
              if (nb[v] + 8 * (j >> 2) + 4 * kg + (j & 3) >= g.N) acc[v][t][j] = -INFINITY;
      }
      // fp32 logits (when asked for) leave first: the statistics below
      // replace each accumulator by exp(x - the lane's maximum), which the
      // fp16 probabilities rescale
      if (!g.p16) store_tile<4, 2>(go, acc, nb, tb, lane);
      float ml[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const MaxSumArg r = lane_stats<4, 2, false, true>(g, acc, nb, t, lane, &ml[t]);
        if (kg == 0) red[wn][rowblk(t) * 32 + r32] = r;
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (tid < kTBT && t0 + tid < g.rows) {
        const MaxSumArg r = msa_merge(red[0][tid], red[1][tid]);
        const int64_t o = int64_t(t0 + tid) * g.n_tiles + n_tile;
        g.t_max[o] = r.m;
        g.t_sum[o] = r.s;
        g.t_arg[o] = r.i;
      }
      if (g.p16) {
        // exp(x - M), M the tile maximum of the token (the value the merge
        // above writes to t_max), as exp(x - m) exp(m - M) with m the lane's
        // maximum (a lane whose columns are all past N stores none of them)
        float sc[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int row = rowblk(t) * 32 + r32;
          const float M = fmaxf(red[0][row].m, red[1][row].m);
          sc[t] = ml[t] == -INFINITY ? 0.f : __expf(ml[t] - M);
        }
        // The tile's fp16 probabilities go through the idle ring (256 rows x
        // 512 B = its 128 KB): each lane writes its 8-byte pieces, 16-byte
        // chunk c of row r at slot c ^ (r & 31) so that a store instruction's
        // 32 rows take distinct banks, then 32 consecutive threads store
        // each row as 16-byte pieces of one 512-byte run (row-strided 8-byte
        // stores straight from the accumulators took about 17 us longer per
        // 256 x 248320 launch, 13 us per 448 x 151936).
        static_assert(kTST * kTSST == kTBT * kTBN * 2, "the fp16 tile fills the ring");
        // the lane's chunk c = 16 wn + 4 v + q of row rl (rl & 31 = r32) sits
        // at slot (16 wn ^ r32) ^ (4 v + q); xs is kept opaque so that the
        // sixteen slot addresses are formed here rather than hoisted out of
        // the tile loop (and spilled)
        int xs = (16 * wn) ^ r32;
        asm volatile("" : "+v"(xs));
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          // (few rows: 32-row blocks past the batch are neither staged nor stored)
          if (SPARSE && rowblk(t) * 32 >= live_rows) continue;
          uint8_t *rowp = smem + (rowblk(t) * 32 + r32) * 512 + kg * 8;
#pragma unroll
          for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              uint32_t hh[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) hh[e] = f2h(acc[v][t][4 * q + e] * sc[t]);
              *reinterpret_cast<uint2 *>(rowp + ((xs ^ (4 * v + q)) << 4)) =
                  make_uint2(hh[0] | (hh[1] << 16), hh[2] | (hh[3] << 16));
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        const int nst = SPARSE ? min(kTBT, live_rows) * 32 : kTBT * 32;
#pragma unroll 4
        for (int i = tid; i < nst; i += 512) {
          const int rl = i >> 5, c = i & 31;
          const int tok = t0 + rl, col = n0 + c * 8;
          if (tok < g.rows && col < g.N)
            *reinterpret_cast<uint4 *>(g.p16 + int64_t(tok) * g.ldo + col) =
                *reinterpret_cast<const uint4 *>(smem + rl * 512 + ((c ^ (rl & 31)) << 4));
        }
      }
    }
    // the staged probabilities are read before the next tile's copies refill the ring
    if (g.p16) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    int next = tile + gridDim.x;
    while (next < n_tiles_all && !valid(next)) next += gridDim.x;
    const bool more = next < n_tiles_all;
    int nn_tile = 0, nt_tile = 0;
    Src nsrc = cur;
    if (more) {
      tile_of(next, nn_tile, nt_tile);
      nsrc = src_of(nn_tile, nt_tile);
#pragma unroll
      for (int p = 0; p < kTST - 1; ++p)
        if (p < nk) issue(nsrc, p);
    }
    if (!more) break;
    tile = next;
    n_tile = nn_tile;
    t_tile = nt_tile;
    cur = nsrc;
  }
}


void launch_gemm_fp8(const GemmArgs &g, hipStream_t s) {
  static bool attr = false;
  static int n_cu = 256;
  if (!attr) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(gemm_fp8_kernel<true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, int(kTiledLds));
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(gemm_fp8_kernel<false>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, int(kTiledLds));
    int dev = 0;
    if (hipGetDevice(&dev) == hipSuccess) {
      int cu = 0;
      if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cu > 0) n_cu = cu;
    }
    attr = true;
  }
  const int n_ntiles = (g.N + kTBN - 1) / kTBN, n_ttiles = (g.rows + kTBT - 1) / kTBT;
  const int tiles = ((n_ntiles + 7) / 8) * 8 * n_ttiles;
  const int grid_x = std::min(tiles, std::max(16, n_cu / 16 * 16));
  // small batches: padding rows are neither fetched nor multiplied (the
  // per-tile checks cost a few percent when every row is live)
  if (g.rows < 128)
    hipLaunchKernelGGL((gemm_fp8_kernel<true>), dim3(grid_x), dim3(512), kTiledLds, s, g);
  else
    hipLaunchKernelGGL((gemm_fp8_kernel<false>), dim3(grid_x), dim3(512), kTiledLds, s, g);
}

// The skinny LM head (<= 32 rows) takes 128 weight rows per workgroup (two
// workgroups per compute unit, 72 KB of LDS each) when 256-row workgroups
// (one per unit, 120 KB) would leave their last dispatch round less than 90 %
// full; otherwise 256 rows, which read the activations half as often.
int lm_tile_width(int rows, int N, int n_cu) {
  if (rows > 64) return kTBN;
  if (rows <= 32) {
    const int64_t tiles = (int64_t(N) + 255) / 256, cu = std::max(n_cu, 1);
    const int64_t rounds = (tiles + cu - 1) / cu;
    if (10 * tiles < 9 * rounds * cu) return 4 * 32;
  }
  return 4 * 2 * 32;
}

// Split-K factor of a projection with `rows` rows: enough workgroups to
// cover the chip, K pieces of at least 256.
int gemm_splits(int rows, int N, int K, int n_cu, int *k_split) {
  int s;
  if (rows <= 64) {
    const int tiles = (N + 127) / 128;
    s = (2 * n_cu + tiles - 1) / tiles;
  } else {
    // the tiled launch pads its grid to a multiple of 8 workgroups (one per
    // CU); every split must fit in one dispatch round
    const int grid_x = ((N + kTBN - 1) / kTBN + 7) / 8 * 8 * ((rows + kTBT - 1) / kTBT);
    s = n_cu / grid_x;
  }
  s = max(1, min(s, K / 256));
  const int ks = ((K + s - 1) / s + 63) / 64 * 64;
  *k_split = ks;
  return (K + ks - 1) / ks;
}

template <int TB, int WV, bool ST>
static void launch_skinny(const GemmArgs &g, int splits, hipStream_t s) {
  constexpr size_t lds = size_t(kSkST) * skinny_stage_bytes<TB, WV>();
  constexpr bool BL = ST;   // the LM head reads the blocked weight copy
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(gemm_skinny_kernel<TB, WV, ST, BL>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    attr = true;
  }
  const dim3 grid((g.N + 4 * WV * 32 - 1) / (4 * WV * 32), splits);
  hipLaunchKernelGGL((gemm_skinny_kernel<TB, WV, ST, BL>), grid, dim3(256), lds, s, g);
}

void launch_gemm_bf16(const GemmArgs &g, bool stats, int splits, hipStream_t s, bool blocked, bool lo) {
  if (g.rows <= 64) {
    // WV = 2 for the LM head (256 weight rows per workgroup), 1 for split-K W_o
    if (g.rows <= 32) {
      if (stats && g.lm_narrow)
        launch_skinny<1, 1, true>(g, splits, s);
      else if (stats)
        launch_skinny<1, 2, true>(g, splits, s);
      else
        launch_skinny<1, 1, false>(g, splits, s);
    } else {
      if (stats) launch_skinny<2, 2, true>(g, splits, s); else launch_skinny<2, 1, false>(g, splits, s);
    }
    return;
  }
  static bool attr_set = false;
  static int n_cu = 256;
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(gemm_tiled_kernel<true, true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, int(kTiledLds));
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(gemm_tiled_kernel<false, false>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, int(kTiledLds));
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(gemm_tiled_kernel<false, true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, int(kTiledLds));
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(gemm_tiled_kernel<false, true, true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, int(kTiledLdsLo));
    int dev = 0;
    if (hipGetDevice(&dev) == hipSuccess) {
      int cu = 0;
      if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cu > 0) n_cu = cu;
    }
    attr_set = true;
  }
  // one workgroup per CU (LDS), a multiple of 16 so that tiles i and i+8 go
  // to co-resident workgroups of one XCD
  const int n_ntiles = (g.N + kTBN - 1) / kTBN, n_ttiles = (g.rows + kTBT - 1) / kTBT;
  const int tiles = ((n_ntiles + 7) / 8) * 8 * n_ttiles;
  const int grid_x = std::min(tiles, std::max(16, n_cu / 16 * 16));
  const dim3 grid(grid_x, splits);
  // the LM head (stats) reads both operands in the blocked layout
  if (stats)
    hipLaunchKernelGGL((gemm_tiled_kernel<true, true>), grid, dim3(512), kTiledLds, s, g);
  else if (blocked && lo)
    hipLaunchKernelGGL((gemm_tiled_kernel<false, true, true>), grid, dim3(512), kTiledLdsLo, s, g);
  else if (blocked)
    hipLaunchKernelGGL((gemm_tiled_kernel<false, true>), grid, dim3(512), kTiledLds, s, g);
  else
    hipLaunchKernelGGL((gemm_tiled_kernel<false, false>), grid, dim3(512), kTiledLds, s, g);
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
  r = msa_wave(r);
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

// One workgroup of 1024 threads per row: each thread sums the split-K
// partials of 4 columns (16-B loads, splits unrolled by 4), keeps h in LDS,
// then scales.
// ----------------------------------------------------------------------------
// FP8 (OCP e4m3) operands: e4m3_code and fp8_exponent come from k_fp8.hpp.
// ----------------------------------------------------------------------------

// 16 consecutive values (already divided by the row scale) -> 16 codes
__device__ __forceinline__ uint4 e4m3_pack16(const float (&v)[16]) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = e4m3_code(v[4 * i]) | (e4m3_code(v[4 * i + 1]) << 8) | (e4m3_code(v[4 * i + 2]) << 16) |
           (e4m3_code(v[4 * i + 3]) << 24);
  return uint4{w[0], w[1], w[2], w[3]};
}

// byte offset of (row, 16-value chunk c16 of the row) in the e4m3 blocked layout
__device__ __forceinline__ int64_t fp8_blocked_off(int64_t row, int c16, int K) {
  const int R = int(row & 255), kb = c16 >> 2, q = c16 & 3;
  return ((row >> 8) * (K >> 6) + kb) * 16384 + R * 64 + (blk_slot(q, R) << 4);
}

// Counts weights that are not finite into *bad (such a row cannot be
// scaled); its codes are still written, from a bounded scale.
__global__ __launch_bounds__(256) void quant_fp8_blocked_kernel(const uint16_t *__restrict__ src,
                                                               uint8_t *__restrict__ dst, float *__restrict__ scale,
                                                               int rows, int K, int32_t *__restrict__ bad) {
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const bool live = row < rows;
  float m = 0.f;
  int n_bad = 0;
  if (live)
    for (int k = tid; k < K; k += 256) {
      const float w = bf2f(src[row * K + k]);
      if (fp8_weight_ok(w))
        m = fmaxf(m, fabsf(w));
      else
        ++n_bad;
    }
  if (n_bad) atomicAdd(bad, n_bad);
  m = wave_max(m);
  __shared__ float red[4];
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  const int e = fp8_exponent(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
  for (int c = tid; c < K / 16; c += 256) {
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = live ? ldexpf(bf2f(src[row * K + c * 16 + i]), -e) : 0.f;
    *reinterpret_cast<uint4 *>(dst + fp8_blocked_off(row, c, K)) = e4m3_pack16(v);
  }
  if (tid == 0) scale[row] = ldexpf(1.0f, e);
}

void launch_quant_fp8_blocked(const uint16_t *src, uint8_t *dst, float *scale, int rows, int K, int32_t *bad,
                              hipStream_t s) {
  const int padded = (rows + 255) / 256 * 256;
  hipLaunchKernelGGL(quant_fp8_blocked_kernel, dim3(padded), dim3(256), 0, s, src, dst, scale, rows, K, bad);
}

__global__ __launch_bounds__(1024) void norm_kernel(const float *part, int splits, int64_t split_stride, int hidden,
                                                    float eps, int mode, void *out, int64_t lo_off, float *a_scale) {
  extern __shared__ float hrow[];     // [hidden]
  const int row = blockIdx.x, tid = threadIdx.x;
  const float *p = part + int64_t(row) * hidden;
  float ss = 0.f;
  for (int c = tid * 4; c < hidden; c += 1024 * 4) {
    f32x4 h4 = {0.f, 0.f, 0.f, 0.f};
    int s = 0;
    for (; s + 4 <= splits; s += 4) {
      const f32x4 a = *reinterpret_cast<const f32x4 *>(p + (s + 0) * split_stride + c);
      const f32x4 b = *reinterpret_cast<const f32x4 *>(p + (s + 1) * split_stride + c);
      const f32x4 d = *reinterpret_cast<const f32x4 *>(p + (s + 2) * split_stride + c);
      const f32x4 e = *reinterpret_cast<const f32x4 *>(p + (s + 3) * split_stride + c);
      h4 = h4 + a;
      h4 = h4 + b;
      h4 = h4 + d;
      h4 = h4 + e;
    }
    for (; s < splits; ++s) h4 = h4 + *reinterpret_cast<const f32x4 *>(p + s * split_stride + c);
    *reinterpret_cast<f32x4 *>(hrow + c) = h4;
    ss = fmaf(h4[0], h4[0], ss);
    ss = fmaf(h4[1], h4[1], ss);
    ss = fmaf(h4[2], h4[2], ss);
    ss = fmaf(h4[3], h4[3], ss);
  }
  ss = wave_sum(ss);
  __shared__ float red[16];
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) tot += red[i];
  const float inv = 1.0f / sqrtf(tot / float(hidden) + eps);
  if (mode == ACT_FP8_BLOCKED) {
    // row scale from the largest |y|, then 16 codes per thread step
    float m = 0.f;
    for (int c = tid; c < hidden; c += 1024) m = fmaxf(m, fabsf(hrow[c] * inv));
    m = wave_max(m);
    __shared__ float redm[16];
    __syncthreads();   // every wave is past its read of red[]
    if ((tid & 63) == 0) redm[tid >> 6] = m;
    __syncthreads();
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, redm[i]);
    const int e = fp8_exponent(amax);
    for (int c = tid; c < hidden / 16; c += 1024) {
      float v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = ldexpf(hrow[c * 16 + i] * inv, -e);
      *reinterpret_cast<uint4 *>(static_cast<uint8_t *>(out) + fp8_blocked_off(row, c, hidden)) = e4m3_pack16(v);
    }
    if (tid == 0) a_scale[row] = ldexpf(1.0f, e);
    return;
  }
  for (int c = tid; c < hidden; c += 1024) {
    const float y = hrow[c] * inv;
    const int64_t idx = int64_t(row) * hidden + c;
    if (mode == ACT_SPLIT) {
      uint16_t hi, lo;
      split_h(y, hi, lo);
      static_cast<uint16_t *>(out)[idx] = hi;
      static_cast<uint16_t *>(out)[lo_off + idx] = lo;
    } else if (mode == ACT_F16) {
      static_cast<uint16_t *>(out)[idx] = f2h(y);
    } else if (mode == ACT_F16_BLOCKED) {
      // the blocked hi plane of the tiled LM head, and the residual y - hi as
      // a row-major fp16 plane at lo_off (the logit refinement reads it)
      uint16_t hi, lo;
      split_h(y, hi, lo);
      const int R = row & 255, q = (c >> 3) & 3;
      const int64_t b = (int64_t(row >> 8) * (hidden >> 5) + (c >> 5)) * 8192;
      static_cast<uint16_t *>(out)[b + R * 32 + (blk_slot(q, R) << 3) + (c & 7)] = hi;
      static_cast<uint16_t *>(out)[lo_off + idx] = lo;
    } else {
      static_cast<float *>(out)[idx] = y;
    }
  }
}

void launch_norm(const float *part, int splits, int64_t split_stride, int rows, int hidden, float eps, int mode,
                 void *out, int64_t lo_off, float *a_scale, hipStream_t s) {
  hipLaunchKernelGGL(norm_kernel, dim3(rows), dim3(1024), size_t(hidden) * 4, s, part, splits, split_stride, hidden,
                     eps, mode, out, lo_off, a_scale);
}


// ----------------------------------------------------------------------------
// weight preparation (once, at handle creation): bf16 -> fp16, round to
// nearest even (exact for 0 and 2^-17 <= |w| <= 65504; see bf8_to_h8).
// Counts values the copy cannot hold (|w| > 65504, infinities, NaN).
// ----------------------------------------------------------------------------

__global__ __launch_bounds__(256) void bf16_to_f16_kernel(const uint16_t *__restrict__ src, uint16_t *__restrict__ dst,
                                                         int64_t n8, int32_t *__restrict__ bad) {
  int local_bad = 0;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n8; i += int64_t(gridDim.x) * 256) {
    const uint4 v = reinterpret_cast<const uint4 *>(src)[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float lo = __uint_as_float(w[k] << 16), hi = __uint_as_float(w[k] & 0xFFFF0000u);
      local_bad += not_f16(lo) + not_f16(hi);
    }
    reinterpret_cast<uint4 *>(dst)[i] = bf8_to_h8(v);
  }
  if (local_bad) atomicAdd(bad, local_bad);
}

// one 16-byte output chunk per thread step: block i >> 10, position i & 1023
__global__ __launch_bounds__(256) void bf16_to_f16_blocked_kernel(const uint16_t *__restrict__ src,
                                                                 uint16_t *__restrict__ dst, int rows, int K,
                                                                 int64_t n16, int32_t *__restrict__ bad) {
  const int kbs = K >> 5;
  int local_bad = 0;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n16; i += int64_t(gridDim.x) * 256) {
    const int64_t blk = i >> 10;
    const int R = int(i >> 2) & 255, p = int(i & 3);
    const int64_t row = (blk / kbs) * 256 + R;
    const int kb = int(blk % kbs), q = blk_slot(p, R);
    uint4 v = {0u, 0u, 0u, 0u};
    if (row < rows) {
      const uint4 b = *reinterpret_cast<const uint4 *>(src + row * K + kb * 32 + q * 8);
      const uint32_t w[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int k = 0; k < 4; ++k)
        local_bad += not_f16(__uint_as_float(w[k] << 16)) + not_f16(__uint_as_float(w[k] & 0xFFFF0000u));
      v = bf8_to_h8(b);
    }
    reinterpret_cast<uint4 *>(dst)[i] = v;
  }
  if (local_bad) atomicAdd(bad, local_bad);
}

void launch_bf16_to_f16_blocked(const uint16_t *src, uint16_t *dst, int rows, int K, int32_t *bad, hipStream_t s) {
  const int64_t n16 = blocked_elems(rows, K) / 8;
  const int64_t blocks = std::min<int64_t>((n16 + 255) / 256, 8192);
  hipLaunchKernelGGL(bf16_to_f16_blocked_kernel, dim3(unsigned(std::max<int64_t>(blocks, 1))), dim3(256), 0, s, src,
                     dst, rows, K, n16, bad);
}

void launch_bf16_to_f16(const uint16_t *src, uint16_t *dst, int64_t n, int32_t *bad, hipStream_t s) {
  const int64_t n8 = n / 8;
  const int64_t blocks = std::min<int64_t>((n8 + 255) / 256, 8192);
  hipLaunchKernelGGL(bf16_to_f16_kernel, dim3(unsigned(std::max<int64_t>(blocks, 1))), dim3(256), 0, s, src, dst, n8,
                     bad);
}

}  // namespace sv
