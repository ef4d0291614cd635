/*
 * spec_verify.h -- C ABI of the MI355X (gfx950) verify step for a parallel
 * draft block.
 *
 * One call scores a whole draft block with the target in one forward pass
 * (sionic.ai "Solar Open2 250B DSpark", section 1: the drafter proposes, the
 * target checks every candidate in one forward, keeps the agreeing leading
 * candidates and restarts at the first difference).  A block is either a
 * chain (the last committed token plus gamma drafts: gamma+1 rows, same
 * page, section 6) or a proposal tree of B anchors x W branch tokens (onedev.kr
 * SpecOPD summary, "how it works" / "what differs": parent map, semantic
 * positions, ancestor-and-self mask).
 *
 * Per row the step computes: RoPE of the row query/key at its semantic
 * position; GQA attention over the tree's KV prefix plus the row's ancestors
 * and itself; W_o; a unit-gain RMS norm; the LM head over the full vocabulary;
 * max / logsumexp / greedy token of the target distribution p; for every
 * non-root row the overlap sum_u min(p_parent(u), q(u)) = 1 - TV(p_parent, q)
 * against the drafter distribution q (SpecOPD summary, "how it is used";
 * VESSL "Speculative Decoding Part 2", DSpark section); the prefix-survival
 * product of overlaps from the root (SpecOPD summary, "how it is used").
 * Per tree it returns the greedy accept length counting the bonus token
 * (SpecOPD summary, "premises and limits"), the bonus token and the last
 * accepted row (VESSL part 2, Blockwise section: keep the longest agreeing
 * prefix).
 *
 * Plain C, no HIP or torch types.  Device pointers are HIP device memory of
 * the current device; `stream` is a hipStream_t passed as void*.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sv_status {
  SV_OK = 0,
  SV_ERR_INVALID_ARG = -1, /* null pointer, bad size or config field      */
  SV_ERR_BAD_TREE = -2,    /* parent map / positions / KV ranges invalid  */
  SV_ERR_CAPACITY = -3,    /* run exceeds a capacity fixed at create       */
  SV_ERR_UNSUPPORTED = -4, /* not a gfx950 device, or unsupported shape    */
  SV_ERR_HIP = -5,         /* a HIP runtime call failed                    */
  SV_ERR_OOM = -6          /* device or pinned host allocation failed      */
} sv_status;

typedef enum sv_dtype { SV_F32 = 0, SV_BF16 = 1 } sv_dtype;

/* Acceptance rule of a run.  SV_MODE_GREEDY: a draft is accepted when it
 * equals the target's greedy token at its parent.  SV_MODE_SAMPLE: T = 1
 * stochastic verification of chains (every row has at most one child): the
 * draft d of row c with parent cur is accepted when u_accept[c] * q_c(d) <
 * p_cur(d), p and q the target and drafter softmaxes; the walk stops at the
 * first rejection and draws the bonus token from max(0, p_cur - q_c), or,
 * after a leaf, from p_cur, by inverse CDF at u_bonus (the smallest token
 * whose running weight exceeds u_bonus times the total weight; from p_cur
 * if the residual has no mass).  The pages evaluate T = 1 sampling
 * (Dev.to/aiwithghost DSpine page, temperature section; SpecOPD summary,
 * "premises and limits") and state its per-position acceptance probability
 * alpha = 1 - D_TV (VESSL part 2, DSpark section), which this rule has. */
typedef enum sv_mode { SV_MODE_GREEDY = 0, SV_MODE_SAMPLE = 1 } sv_mode;

/* Number format of the LM head.  SV_WEIGHTS_NATIVE: cfg->dtype (bf16 weights
 * run as exact fp16 copies, fp32 as given).  SV_WEIGHTS_FP8 (bf16 models
 * only): W8A8 in OCP e4m3, as the pages' fastest serving runs the target in
 * FP8 (sionic.ai "Solar Open2 250B DSpark", section 5).  Each LM-head row n
 * and each normalised hidden row t is divided by a power of two, s_n = 2^e
 * with e the smallest integer such that max |row| <= 448 * 2^e (1 for a zero
 * row), and rounded to the nearest e4m3 value (ties to even); logits[t, n] =
 * a_t s_n sum_k q_h[t, k] q_w[n, k], accumulated in fp32.  Exponents below
 * -126 are raised to -126, so that every scale is a normal fp32 number.  W_o
 * stays in the native format. */
typedef enum sv_weights { SV_WEIGHTS_NATIVE = 0, SV_WEIGHTS_FP8 = 1 } sv_weights;

/* Model shape and capacities, fixed for the handle's lifetime. */
typedef struct sv_config {
  int32_t n_q_heads;     /* Hq; a multiple of n_kv_heads                       */
  int32_t n_kv_heads;    /* Hkv; query head h reads KV head h / (Hq/Hkv)       */
  int32_t head_dim;      /* d: 64, 128 or 256                                  */
  int32_t hidden;        /* model width (W_o rows, LM-head columns); % 64 == 0 */
  int32_t vocab;         /* V >= 2                                             */
  int32_t dtype;         /* sv_dtype of KV, row q/k/v, weights, drafter logits */
  float rope_base;       /* RoPE base (10000); NeoX half-split pairs (k,k+d/2)  */
  float norm_eps;        /* final RMS-norm epsilon (1e-6), unit gain           */
  int32_t max_rows;      /* most rows in one run                              */
  int32_t max_roots;     /* most trees in one run                             */
  int32_t max_tree_rows; /* most rows in one tree, <= 64                      */
  int32_t max_pos;       /* every semantic position must be < max_pos         */
  int32_t weight_format; /* sv_weights of the LM head; 0 when zero-initialised */
} sv_config;

typedef struct sv_handle sv_handle;

/* One verify step.  Trees are contiguous row ranges, each starting with its
 * root (parent -1); for a non-root row i of the tree starting at s,
 * s <= parent[i] < i.  Roots are numbered in row order and index the
 * root_kv_* arrays.  Non-root ("draft") rows are numbered in row order and
 * index drafter_logits.
 *
 * Device buffers: kv_k, kv_v, q_rows, k_rows, v_rows, drafter_logits (and
 * the outputs' logits) must be 16-byte aligned, the other device arrays
 * 4-byte aligned (SV_ERR_INVALID_ARG otherwise, before anything is
 * enqueued).  A draft id may be any int32: one outside [0, V) is a token
 * neither model can emit, so it is never accepted (in SV_MODE_SAMPLE its
 * target probability is 0), and nothing is read for it. */
typedef struct sv_inputs {
  int32_t n_rows;              /* 1 .. max_rows                                 */
  int32_t n_roots;             /* number of trees (rows with parent -1)         */
  const int32_t *parent;       /* HOST   [n_rows]                               */
  const int32_t *pos;          /* HOST   [n_rows]  semantic positions, 0..max_pos-1 */
  const int64_t *root_kv_off;  /* HOST   [n_roots] first visible prefix token   */
  const int32_t *root_kv_len;  /* HOST   [n_roots] visible prefix length (>= 0) */
  int64_t kv_tokens;           /* tokens in kv_k / kv_v                         */
  const void *kv_k;            /* DEVICE [kv_tokens, Hkv, d], keys already rotated */
  const void *kv_v;            /* DEVICE [kv_tokens, Hkv, d]                    */
  const void *q_rows;          /* DEVICE [n_rows, Hq, d]  queries before RoPE   */
  const void *k_rows;          /* DEVICE [n_rows, Hkv, d] keys before RoPE      */
  const void *v_rows;          /* DEVICE [n_rows, Hkv, d]                       */
  const int32_t *draft_ids;    /* DEVICE [n_rows] token at each row; roots ignored; see above for ids outside [0, V) */
  const void *drafter_logits;  /* DEVICE [n_rows - n_roots, V]                  */
  int32_t mode;                /* sv_mode; 0 (greedy) when zero-initialised     */
  const float *u_accept;       /* DEVICE [n_rows] uniforms in [0, 1), SV_MODE_SAMPLE only; roots ignored */
  const float *u_bonus;        /* DEVICE [n_roots] uniforms in [0, 1), SV_MODE_SAMPLE only */
} sv_inputs;

/* Outputs, all DEVICE memory written by the run.  `logits` may be NULL. */
typedef struct sv_outputs {
  int32_t *accept_len;  /* [n_roots] accepted drafts + 1 (bonus), in [1, depth+1] */
  int32_t *bonus;       /* [n_roots] bonus token: greedy token of the last accepted
                           row, or (SV_MODE_SAMPLE) the draw described at sv_mode */
  int32_t *last_row;    /* [n_roots] last accepted row (global row index)           */
  float *surv_sum;      /* [n_roots] sum of survival over the tree's non-root rows  */
  int32_t *argmax;      /* [n_rows] greedy token (lowest id among equal maxima)     */
  float *row_max;       /* [n_rows] max logit                                       */
  float *row_lse;       /* [n_rows] log sum exp of the logits                       */
  float *overlap;       /* [n_rows] sum_u min(p_parent, q); 1 for roots             */
  float *survival;      /* [n_rows] product of overlaps root..row; 1 for roots      */
  float *logits;        /* [n_rows, V] fp32 target logits, or NULL                  */
} sv_outputs;

/* Create a handle on the current device.  w_o is DEVICE [hidden, Hq*d] and
 * w_lm is DEVICE [vocab, hidden], both row-major in cfg->dtype.  For SV_BF16
 * the handle converts them once into fp16 copies it owns, rounding to
 * nearest even: exact for 0 and every bf16 value with 2^-17 <= |w| <=
 * 65504, smaller magnitudes become the nearest multiple of 2^-24; a weight
 * above 65504 in magnitude, infinite or NaN fails with SV_ERR_UNSUPPORTED.
 * With SV_WEIGHTS_FP8, W_lm becomes e4m3 codes and row scales instead (a
 * weight that is not finite fails with SV_ERR_UNSUPPORTED).  The caller's
 * bf16 buffers are not used after create returns; for SV_F32 they are
 * borrowed for the handle's lifetime.  Allocates the handle's device scratch
 * (sized from the capacities) and pinned host staging; synchronises the
 * device.  Fails with SV_ERR_UNSUPPORTED unless the device is gfx950. */
sv_status spec_verify_create(const sv_config *cfg, const void *w_o, const void *w_lm,
                             sv_handle **out);

/* Enqueue one verify step on `stream` (hipStream_t; NULL = default stream).
 * in->mode selects the acceptance rule (sv_mode); SV_MODE_SAMPLE needs
 * u_accept and u_bonus and fails with SV_ERR_UNSUPPORTED when a row has
 * more than one child.
 * Host arrays are read and copied before the call returns; device inputs and
 * outputs must stay valid until the stream passes the enqueued work.  The
 * step's metadata goes through one of 4 pinned staging slots of the handle,
 * used in turn: the call waits on the host only until the device has
 * finished the metadata copy of the run 4 calls back on this handle, whose
 * slot it reuses (so at most 4 runs of a handle are queued ahead of the
 * device; with fewer queued the call never waits).  Every
 * argument, tree, alignment and capacity check happens before anything is
 * enqueued: on error nothing was enqueued and the outputs are untouched.  A
 * handle runs one step at a time: steps on one handle must be ordered by the
 * caller (same stream, or events). */
sv_status spec_verify_run(sv_handle *h, const sv_inputs *in, const sv_outputs *out, void *stream);

/* Commit of the handle's most recent step: the step after verify, which keeps
 * the accepted drafts and resumes after them (sionic.ai "Solar Open2 250B
 * DSpark", section 1; section 6 names committing accepted tokens as the part
 * of the loop that follows verify).  For tree t with visible prefix
 * [root_kv_off[t], root_kv_off[t] + root_kv_len[t]), the accepted path -- the
 * root, then every accepted draft in depth order, accept_len[t] rows ending at
 * last_row[t] -- is written to cache entries root_kv_off[t] + root_kv_len[t]
 * + j, j = 0 .. accept_len[t] - 1: K = the row key rotated at its semantic
 * position (as the step computed it), V = the row value, both in cfg->dtype.
 * Paths through a tree are compacted this way.  The bonus token is not
 * written: it is the next step's root, at the position after the last
 * committed row, seeing root_kv_len[t] + accept_len[t] entries.
 *
 * `in` and `out` are those of the most recent spec_verify_run on this handle
 * (same host arrays, same v_rows; accept_len and last_row are read on the
 * device, so the host does not wait), and `stream` is that run's stream:
 * otherwise SV_ERR_INVALID_ARG.  kv_k and kv_v are the cache, DEVICE
 * [in->kv_tokens, Hkv, d], writable, 16-byte aligned (normally the run's
 * in->kv_k and in->kv_v).  SV_ERR_BAD_TREE when some tree's possible write
 * range [off + len, off + len + depth + 1), depth = its deepest row, leaves
 * [0, kv_tokens) or overlaps another tree's visible prefix or write range (a
 * shared stem cannot take commits).  Enqueues one kernel; never synchronises.
 * The next spec_verify_run on the handle replaces what a later commit would
 * read. */
sv_status spec_verify_commit(sv_handle *h, const sv_inputs *in, const sv_outputs *out, void *kv_k, void *kv_v,
                             void *stream);

/* Verify budget over a batch of requests: which draft candidates each request
 * verifies in the next step.  A confidence head's per-position pass
 * probabilities, multiplied along a path, give the probability that the
 * position is accepted; the batch's verify budget goes to the positions most
 * likely to pass, across all requests, to maximise throughput on a measured
 * hardware curve, so gamma varies per request and with load (VESSL AI
 * "Speculative Decoding Part 2", DSpark section; branch scores as path
 * products, EAGLE-2, same page).
 *
 * Request r offers n_cand[r] >= 0 candidates; the candidate arrays hold the
 * requests one after another.  cand_parent[k] is the candidate (request-local
 * index, earlier than k) that candidate k follows, or -1 for the request's
 * last committed token (its verify root); cand_conf[k] in [0, 1] is the
 * probability that k passes given that its parent passed (a chain: parent k-1).
 * A candidate's score is the product of conf along its path.  Every request
 * verifies its root, so selecting m candidates makes a step of n_req + m rows
 * with expected n_req + (sum of their scores) committed tokens.  Step times
 * come from the measured curve (curve_rows strictly increasing, curve_ms
 * positive and non-decreasing): linear between points, the first value below
 * the first point, extended from the last two points past the last.  The call
 * selects the candidates that maximise expected tokens per ms -- the m highest
 * scores (ties: earlier request, then earlier candidate; this keeps each
 * selected candidate's parent selected) for the best m, the smallest m on ties
 * -- with at most max_rows rows when max_rows > 0.
 *
 * HOST memory only, no GPU work, no handle.  selected[k] (int32 per
 * candidate) is set to 1 or 0; *expected_tokens and *step_ms (may be NULL)
 * receive the chosen step's figures.  SV_ERR_INVALID_ARG for bad counts,
 * confidences or curve, SV_ERR_BAD_TREE for a bad parent, SV_ERR_CAPACITY when
 * max_rows is below n_req. */
sv_status spec_verify_schedule(int32_t n_req, const int32_t *n_cand, const int32_t *cand_parent,
                               const float *cand_conf, int32_t n_curve, const int32_t *curve_rows,
                               const float *curve_ms, int32_t max_rows, int32_t *selected,
                               double *expected_tokens, double *step_ms);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): one verify
 * step of an fp32 model (cfg->dtype SV_F32, native weights) without a handle.
 * w_o and w_lm are DEVICE [hidden, Hq*d] and [vocab, hidden] fp32, used as
 * given; cfg, in and out mean what they mean for spec_verify_create and
 * spec_verify_run, and every check of those calls happens before anything is
 * enqueued.  The call allocates no device, pinned or managed memory: every
 * per-run buffer (metadata, rotated rows, attention output, hidden rows,
 * logits when out->logits is NULL, tile and chunk records) lives in one
 * 8 MiB array of the library, which every device it runs on holds until the
 * process ends; a run that needs more fails with SV_ERR_CAPACITY (the logits
 * take rows x vocab x 4 bytes unless the caller passes a logits buffer).  The
 * step's metadata travels as kernel arguments, so host arrays may be reused
 * as soon as the call returns; host-side planning uses ordinary heap memory
 * of a few KB.  All calls on one device share that device's array, which
 * keeps the last call's contents: calls that overlap on one device race, so
 * the caller orders them (one stream, or events).  Enqueues on `stream`
 * (hipStream_t; NULL = default) and never waits on the host.  Fails with
 * SV_ERR_UNSUPPORTED for other dtypes, weight formats or devices. */
sv_status spec_verify_run_static(const sv_config *cfg, const void *w_o, const void *w_lm, const sv_inputs *in,
                                 const sv_outputs *out, void *stream);

/* Prepared weights, for callers that convert a bf16 model's weights once and
 * share them between handles (a bf16 handle made by spec_verify_create keeps
 * its own fp16 copies: about 2.5 GB for a 248320 x 5120 LM head).  The three
 * calls below are for cfg->dtype SV_BF16 with weight_format
 * SV_WEIGHTS_NATIVE; any other cfg fails with SV_ERR_UNSUPPORTED.
 *
 * spec_verify_weight_bytes: HOST only, no GPU work.  *bytes receives the size
 * of one device buffer that holds W_o as fp16 row-major, W_o and W_lm in
 * the blocked fp16 layout of the tiled launches, and a 256-byte check word.
 * The size depends on hidden, n_q_heads * head_dim and vocab only, not on the
 * capacities, so one buffer serves handles of any capacities.
 *
 * spec_verify_prepare_weights: converts the bf16 weights w_o and w_lm
 * (DEVICE, as for spec_verify_create) into dst (DEVICE, caller-owned,
 * spec_verify_weight_bytes bytes, 256-byte aligned) on `stream`, then WAITS
 * for the conversion.  The conversion rounds to nearest even, exactly as
 * spec_verify_create's does.  Fails with SV_ERR_UNSUPPORTED when a weight is
 * not finite or exceeds 65504 in magnitude; dst is then unusable.
 *
 * spec_verify_create_prepared: as spec_verify_create, but the handle borrows
 * `prepared` (a buffer filled by spec_verify_prepare_weights for a cfg with
 * the same hidden, n_q_heads, head_dim and vocab) instead of copying the
 * weights.  The caller keeps it alive and unchanged until the handle is
 * destroyed; the library never frees it.  Results are identical to those of
 * a handle made by spec_verify_create from the same bf16 weights. */
sv_status spec_verify_weight_bytes(const sv_config *cfg, size_t *bytes);
sv_status spec_verify_prepare_weights(const sv_config *cfg, const void *w_o, const void *w_lm, void *dst,
                                      void *stream);
sv_status spec_verify_create_prepared(const sv_config *cfg, const void *prepared, sv_handle **out);

/* Wait for the handle's last enqueued step, then free everything it owns.
 * NULL is accepted. */
sv_status spec_verify_destroy(sv_handle *h);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char *spec_verify_last_error(void);

/* Per-stage device times, for profiling.  spec_verify_profile(h, mode)
 * drops earlier records and sets what later runs record on their stream:
 * mode 1, a HIP event before and after each stage and around the whole step
 * (stage "step"); mode 2, events around the LM-head stage only (the step's
 * dominant kernel, at the cost of two events per run); mode 0, nothing.
 * Other modes fail with SV_ERR_INVALID_ARG.  spec_verify_stage_times waits
 * for the last recorded run, then writes up to `cap` stage names (static
 * strings) and their mean duration in ms over all runs recorded since the
 * mode was set; returns the number of stages (0 if nothing was recorded), or
 * a negative sv_status. */
sv_status spec_verify_profile(sv_handle *h, int32_t mode);
int32_t spec_verify_stage_times(sv_handle *h, const char **names, float *ms, int32_t cap);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
