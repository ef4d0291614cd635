// Kernel argument blocks and host-side launchers of the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.hpp"

namespace sv {

// Formats of the projections' small (activation) operand: ACT_SPLIT = fp16
// hi plane + fp16 lo plane (hi + lo = value to ~22 bits), ACT_F16, ACT_F32,
// ACT_F16_BLOCKED = fp16 in the blocked layout below, ACT_SPLIT_BLOCKED = the
// hi and lo planes, each in the blocked layout (W_o above 64 rows).
enum ActMode : int {
  ACT_SPLIT = 0,
  ACT_F16 = 1,
  ACT_F32 = 2,
  ACT_F16_BLOCKED = 3,
  ACT_FP8_BLOCKED = 4,
  ACT_SPLIT_BLOCKED = 5
};

// FP8 (OCP e4m3) operands of the FP8 LM head: each row of W and of the
// activations is stored as e4m3 codes of value / 2^e, 2^e the smallest
// power of two with max |row| <= 448 * 2^e, in a blocked layout like the fp16
// one with K steps of 64 (64 bytes per row): blocks [rows / 256][K / 64] of
// 256 x 64 bytes, 16-byte chunk q of row R at byte R * 64 + (blk_slot(q, R)
// << 4).  The scales 2^e are kept per row as floats.

// Blocked fp16 layout of a [M, K] operand of the tiled LM-head launch: rows
// padded to a multiple of 256; blocks [M / 256][K / 32], each 256 rows x 64
// bytes (one K step) = 16 KB.  Inside a block, row R's 16-byte chunk q
// (elements 8q .. 8q+7 of the K step) sits at byte R * 64 + (blk_slot(q, R)
// << 4): the image of one ring stage in LDS, so that every DMA instruction
// reads 1 KB of consecutive bytes.
constexpr int64_t blocked_elems(int64_t rows, int64_t K) { return (rows + 255) / 256 * 256 * K; }

// Slot of 16-byte chunk q (0..3) of row R in a 64-byte row of a blocked
// stage.  Sixteen consecutive rows put one chunk in sixteen distinct
// 16-byte bank groups of a 256-byte LDS line, so a 16-byte fragment read of
// 32 consecutive rows (one MFMA operand) runs without bank conflicts.
__host__ __device__ constexpr int blk_slot(int q, int R) { return q ^ ((R >> 2) & 3); }

struct AttnArgs {
  const uint16_t *kv_k, *kv_v;     // [T, Hkv, D] bf16, keys already rotated
  const uint16_t *k_rot, *v_rows;  // [n, Hkv, D] bf16, row keys rotated (hi plane)
  const uint16_t *q_rot;           // [n, Hq, D] bf16 hi plane of the rotated queries
  int64_t q_lo_off;                // elements from the hi plane to the lo plane
  const AttnItem *items;
  const AttnRun *runs;             // one per workgroup
  const uint64_t *row_panc;        // [n] ancestor-or-self bits relative to the row's pack
  const int32_t *row_klen;         // [n] prefix keys the row sees (its tree's length)
  float *part_o, *part_ml;         // [slots, D], [slots, 2]
  int Hq, Hkv, G;
  float scale_log2;                // log2(e) / sqrt(D)
  int nt_part;                     // 1: o records stored with the non-temporal hint
};

struct MergeArgs {
  const float *part_o, *part_ml;
  const AttnGroup *groups;         // [R * Hkv * qg_max], by pack
  const int32_t *row_tree, *row_local;   // the row's pack and its row within the pack
  int Hq, Hkv, qg_max;
  int mode;                        // ACT_SPLIT: fp16 hi plane at out, lo at out + lo_off; ACT_F16; ACT_F16_BLOCKED
  int64_t lo_off;
  uint16_t *out;                   // [n, Hq*D]
  // exact weights of the keys rotated in this step (bf16 path): the row's
  // ancestor-or-self bits in its own tree, its tree and the trees' first
  // rows, the rotated queries and keys (hi planes, lo planes at q_lo_off /
  // k_lo_off), the row values, the score scale in log2 units.  row_anc null:
  // off.
  const uint64_t *row_anc;
  const int32_t *row_tree_real, *tree_start;
  const uint16_t *q_rot, *k_rot, *v_rows;
  int64_t q_lo_off, k_lo_off;
  float scale_log2;
};

struct AttnF32Args {
  const float *kv_k, *kv_v, *k_rot, *v_rows, *q_rot;
  const int32_t *row_tree, *tree_start, *tree_rows, *tree_kv_len;
  const int64_t *tree_kv_off;
  const uint64_t *row_anc;
  float *out;                      // [n, Hq*D]
  int Hq, Hkv, D;
};

// out[rows, N] = act[rows, K] . W[N, K]^T, W in fp16, fp32 accumulation.
// rows <= 64: act is an fp16 hi + lo pair (ACT_SPLIT); rows > 64: fp16.  The
// stats launch (the LM head) reads W in the blocked layout, and for rows > 64
// act too; otherwise both are row-major.
// Split-K (grid.y) writes out + split * split_stride.  With stats, each
// workgroup also writes (max, sum exp(x - max), argmax) of its N tile per row.
struct GemmArgs {
  const uint16_t *act;             // skinny: fp16 hi plane; tiled: fp16
  const uint16_t *act_lo;          // skinny: fp16 lo plane

  int rows;
  const uint16_t *W;
  int N, K;
  int k_split;
  float *out;
  int64_t ldo, split_stride;
  float *t_max, *t_sum;
  int32_t *t_arg;
  int n_tiles;
  // tiled LM head: when non-null, the tile's probabilities relative to its
  // maximum, exp(l - t_max), as fp16 [rows, ldo], replace the fp32 logits
  uint16_t *p16;
  // skinny LM head: 128 weight rows per workgroup (lm_tile_width said 128)
  int lm_narrow;
  // FP8 LM head: e4m3 operands in the blocked layout and their row scales
  const uint8_t *W8, *act8;
  const float *w_scale, *a_scale;
};

// ---- attention ----
void launch_rope_f32(const float *q, const float *k, float *qo, float *ko, const int32_t *row_pos, int n, int Hq,
                     int Hkv, int D, double base, hipStream_t s);
void launch_attn_mfma(const AttnArgs &a, int n_runs, int D, int max_qblocks, hipStream_t s);
void launch_attn_merge(const MergeArgs &a, int n_rows, int D, double mean_items, hipStream_t s);
void launch_attn_f32(const AttnF32Args &a, int n_rows, hipStream_t s);

// ---- projections ----
// Tile width (N columns per stats record) of the LM-head launch chosen for
// `rows` rows, N columns and n_cu compute units.
int lm_tile_width(int rows, int N, int n_cu);
// Split-K factor (and K per split, a multiple of 64) of a projection launch.
int gemm_splits(int rows, int N, int K, int n_cu, int *k_split);
// `blocked`: the tiled launch reads W and act in the blocked layout (always
// for stats, the LM head)
// `lo` (with `blocked`, not the LM head): act is an fp16 hi plane at g.act and
// a lo plane at g.act_lo, both blocked; two MFMAs per product.
void launch_gemm_bf16(const GemmArgs &g, bool stats, int splits, hipStream_t s, bool blocked = false,
                      bool lo = false);
void launch_gemm_f32(const float *act, int rows, const float *W, int N, int K, float *out, hipStream_t s);
void launch_stats_from_logits(const float *logits, int rows, int V, int tile, float *t_max, float *t_sum,
                              int32_t *t_arg, int n_tiles, hipStream_t s);
// Writes the normalised rows in `mode` (ACT_SPLIT: fp16 hi plane at out, lo
// plane at out + lo_off; ACT_F16; ACT_F32; ACT_F16_BLOCKED; ACT_FP8_BLOCKED,
// with each row's scale at a_scale[row]).
void launch_norm(const float *part, int splits, int64_t split_stride, int rows, int hidden, float eps, int mode,
                 void *out, int64_t lo_off, float *a_scale, hipStream_t s);
// FP8 LM head: logits and tile statistics like the stats launch, from g.W8,
// g.act8, g.w_scale, g.a_scale (any row count).
void launch_gemm_fp8(const GemmArgs &g, hipStream_t s);
// bf16 [rows, K] row-major -> e4m3 blocked layout (blocked_elems(rows, K)
// bytes, K % 64 == 0) and scale[] (rows padded to 256; padding rows: codes 0,
// scale 1).  Adds the count of weights that are not finite to *bad.
void launch_quant_fp8_blocked(const uint16_t *src, uint8_t *dst, float *scale, int rows, int K, int32_t *bad,
                              hipStream_t s);

// bf16 -> fp16 copy of n values (n % 8 == 0); adds the count of values
// outside the fp16 range to *bad (device int).
void launch_bf16_to_f16(const uint16_t *src, uint16_t *dst, int64_t n, int32_t *bad, hipStream_t s);
// bf16 [rows, K] row-major -> fp16 blocked layout (blocked_elems(rows, K)
// values, padding rows zero); K % 32 == 0.  Adds the count of values outside
// the fp16 range to *bad.
void launch_bf16_to_f16_blocked(const uint16_t *src, uint16_t *dst, int rows, int K, int32_t *bad, hipStream_t s);

// ---- vocabulary reductions and acceptance ----
struct VocabArgs {
  int n, n_draft, R, V;
  const int32_t *row_parent, *row_draft, *draft_row, *tree_start, *tree_rows;
  const int32_t *row_tree;      // [n] tree of each row
  int32_t *tree_done;           // [R] completion counters (zero at the start of a run)
  const int32_t *draft_ids;
  const void *drafter;          // [n_draft, V] bf16 or f32
  int drafter_bf16;
  float *logits;                // [n, V] fp32 (the refinement rewrites some entries)
  // [n, V] fp16 exp(l - t_max) per LM-head tile (null: read `logits`)
  uint16_t *p16;
  const float *t_max, *t_sum;
  const int32_t *t_arg;
  int n_tiles;
  int tile_shift;               // log2 of the LM head's tile width (8, or 7 for 128-token tiles)
  float2 *dpart;                // [n_draft, n_dch]
  int n_dch, dchunk;
  float *lse_q;                 // [n_draft]
  float *opart;                 // [n_draft, n_och]
  int n_och, ochunk;
  // outputs
  int32_t *argmax, *accept_len, *bonus, *last_row;
  float *row_max, *row_lse, *overlap, *survival, *surv_sum;
  // Logit refinement of the tiled LM head (plain fp16 activations): the
  // row statistics recompute every token with probability >= 1/64 from the
  // fp16 hi + lo activation pair.  rf_w: LM-head weights (blocked fp16),
  // rf_hi: the rows' blocked fp16 activations, rf_lo: their row-major fp16
  // residuals, rf_K: hidden width.  rf_w null: off.
  const uint16_t *rf_w, *rf_hi, *rf_lo;
  int rf_K;
};
// T = 1 stochastic verification of chains (see sv_mode in spec_verify.h).
struct SampleArgs {
  const int32_t *row_child;     // [n] the row's child or -1
  const float *u_accept;        // [n]
  const float *u_bonus;         // [R]
  int32_t *rej_child;           // [R] rejected child of the stop row, -1 after a leaf
  float *rpart;                 // [R, n_och] canonical chunk sums of the bonus weights
};
void launch_sample(const VocabArgs &a, const SampleArgs &sa, hipStream_t s);

// ---- commit (the step after verify) ----
// Tree t's accepted path (root first, accept_len[t] rows ending at
// last_row[t]) is copied to cache entries kv_off[t] + kv_len[t] + j: K from
// the run's rotated row keys, V from the row values; row_bytes per KV row.
struct CommitArgs {
  const int32_t *row_parent;    // [n] global parent row, -1 for roots
  const int32_t *tree_start, *tree_rows;
  const int32_t *accept_len, *last_row;   // [R] outputs of the run
  const int64_t *kv_off;        // [R] the tree's first visible cache entry
  const int32_t *kv_len;        // [R] visible prefix length
  const uint8_t *k_rot, *v_rows;          // [n] rows of row_bytes
  uint8_t *kv_k, *kv_v;         // cache, rows of row_bytes
  int row_bytes;                // Hkv * d * element size, a multiple of 16
};
void launch_commit(const CommitArgs &a, int n_roots, hipStream_t s);

void launch_drafter_partial(const VocabArgs &a, hipStream_t s);
// bf16 RoPE of the rows (as launch_rope_bf16) and the drafter statistics (as
// launch_drafter_partial) in one launch; ry = ceil((Hq + Hkv) * D / 2 / 256).
struct RopeArgs {
  const uint16_t *q, *k;
  uint16_t *q_out, *k_out;
  const int32_t *row_pos;
  int Hq, Hkv, D;
  double base;
  int64_t q_lo_off, k_lo_off;      // lo planes of the rotated queries and keys
  int n, ry;
};
void launch_rope_drafter_bf16(const RopeArgs &r, const VocabArgs &a, hipStream_t s);
// row_combine and overlap_partial in one launch (small batches: each
// overlap workgroup recomputes its two logsumexps from the tile records)
void launch_combine_overlap(const VocabArgs &a, hipStream_t s);
// Largest combine_overlap launch that also runs the acceptance walks, and
// whether this one does (otherwise launch_accept follows it).
constexpr int kFusedAcceptMaxBlocks = 256;
bool combine_overlap_accepts(const VocabArgs &a);
void launch_row_combine(const VocabArgs &a, hipStream_t s);
void launch_overlap_partial(const VocabArgs &a, hipStream_t s);
void launch_accept(const VocabArgs &a, hipStream_t s);

}  // namespace sv
