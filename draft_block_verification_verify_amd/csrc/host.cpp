// C ABI of the verify step (include/spec_verify.h): handle lifetime, scratch,
// weight preparation (fp16 or e4m3 copies), metadata upload and the launch
// sequence of one run, the commit of a run's accepted paths, and the
// host-only verify-budget schedule.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "launch.hpp"
#include "plan.hpp"
#include "schedule.hpp"
#include "spec_verify.h"

namespace {

thread_local std::string g_err;

sv_status fail(sv_status st, std::string msg) {
  g_err = std::move(msg);
  return st;
}

constexpr int kRing = 4;          // pinned metadata staging slots
constexpr int kDChunk = 2048;     // vocabulary chunk of the drafter-stats pass (one record per wavefront)
constexpr int kOChunk = 8192;     // vocabulary chunk of the overlap pass and of the T = 1 draw

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Stage {
  const char *name;
  hipEvent_t a, b;
};

}  // namespace

struct sv_handle {
  sv_config cfg{};
  sv::Dims dm{};
  // weights the kernels read: for bf16, fp16 copies (W_o row-major, W_lm in
  // the blocked layout of the LM-head launches)
  const void *w_o = nullptr, *w_lm = nullptr;
  const void *w_o_blk = nullptr;   // bf16, max_rows > 64: W_o in the blocked layout of the tiled launch
  // FP8 LM head: e4m3 W_lm (blocked) and its row scales; per-run row scales
  // of the activations
  uint8_t *w_lm8 = nullptr;
  float *w_scale = nullptr, *a_scale = nullptr;
  int32_t *d_bad = nullptr;
  int device = 0, n_cu = 256, target_items = 1024;
  int elt = 2;
  // metadata
  char *d_meta = nullptr;
  size_t meta_cap = 0;
  char *h_meta[kRing] = {};
  hipEvent_t meta_ev[kRing] = {};
  bool meta_used[kRing] = {};
  int ring = 0;
  // scratch
  void *q_rot = nullptr, *k_rot = nullptr, *o_act = nullptr, *hn = nullptr;
  float *part_o = nullptr, *part_ml = nullptr, *h_part = nullptr, *logits = nullptr;
  float *t_max = nullptr, *t_sum = nullptr, *lse_q = nullptr, *opart = nullptr;
  uint16_t *p16 = nullptr;         // LM head: fp16 tile-relative probabilities
  int32_t *t_arg = nullptr;
  float2 *dpart = nullptr;
  int64_t slot_cap = 0;
  int n_tiles_cap = 0, n_dch = 0, n_och = 0;
  int32_t *rej_child = nullptr;    // T = 1 mode: per tree
  float *rpart = nullptr;          // T = 1 mode: [max_roots, n_och]
  size_t h_part_floats = 0;
  std::vector<void *> allocs;
  // the most recent run, for spec_verify_commit (its plan stays in d_meta
  // until the next run's upload, which is ordered after the commit on the
  // same stream)
  struct LastRun {
    bool valid = false;
    void *stream = nullptr;
    int32_t n = 0, R = 0;
    int64_t kv_tokens = 0;
    const void *v_rows = nullptr;
    std::vector<int32_t> parent, pos, kv_len, depth;   // depth: deepest row of each tree
    std::vector<int64_t> kv_off;
    sv::MetaLayout lay{};
  } last;
  // completion / profiling
  hipEvent_t done = nullptr;
  bool ran = false;
  int profile = 0;                 // 0 off, 1 every stage, 2 the LM head only
  std::vector<Stage> stages;      // every recorded stage of every recorded run
};

namespace {

sv_status hip_fail(const char *what, hipError_t e) {
  return fail(SV_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

template <class T>
sv_status dev_alloc(sv_handle *h, T **p, size_t bytes) {
  void *q = nullptr;
  if (bytes == 0) bytes = 16;
  const hipError_t e = hipMalloc(&q, bytes);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(SV_ERR_OOM, "hipMalloc of " + std::to_string(bytes) + " bytes failed: " + hipGetErrorString(e));
  }
  h->allocs.push_back(q);
  *p = static_cast<T *>(q);
  return SV_OK;
}

void release(sv_handle *h) {
  for (void *p : h->allocs) (void)hipFree(p);
  h->allocs.clear();
  for (int i = 0; i < kRing; ++i) {
    if (h->h_meta[i]) (void)hipHostFree(h->h_meta[i]);
    if (h->meta_ev[i]) (void)hipEventDestroy(h->meta_ev[i]);
  }
  if (h->done) (void)hipEventDestroy(h->done);
  for (auto &s : h->stages) {
    (void)hipEventDestroy(s.a);
    (void)hipEventDestroy(s.b);
  }
  h->stages.clear();
  delete h;
}

// Scratch buffers of the vocabulary stages of one run.
struct VocabBufs {
  float *logits;
  uint16_t *p16;
  float *t_max, *t_sum;
  int32_t *t_arg;
  int n_tiles;
  float2 *dpart;
  int n_dch;
  float *lse_q, *opart;
  int n_och;
};

// Arguments of the vocabulary stages (statistics, overlaps, acceptance, the
// T = 1 draw) of one run, from its plan, its device metadata and buffers.
sv::VocabArgs vocab_args(const sv::Plan &plan, const char *m, const sv::MetaLayout &lay, int V, bool bf16,
                         const sv_inputs *in, const sv_outputs *out, const VocabBufs &b) {
  sv::VocabArgs va{};
  va.tile_shift = 8;
  va.n = plan.n;
  va.n_draft = plan.n_draft;
  va.R = plan.R;
  va.V = V;
  va.row_parent = reinterpret_cast<const int32_t *>(m + lay.row_parent);
  va.row_draft = reinterpret_cast<const int32_t *>(m + lay.row_draft);
  va.draft_row = reinterpret_cast<const int32_t *>(m + lay.draft_row);
  va.tree_start = reinterpret_cast<const int32_t *>(m + lay.tree_start);
  va.tree_rows = reinterpret_cast<const int32_t *>(m + lay.tree_rows);
  va.row_tree = reinterpret_cast<const int32_t *>(m + lay.row_tree);
  va.tree_done = reinterpret_cast<int32_t *>(const_cast<char *>(m) + lay.tree_done);
  va.draft_ids = in->draft_ids;
  va.drafter = in->drafter_logits;
  va.drafter_bf16 = bf16 ? 1 : 0;
  va.logits = b.logits;
  va.p16 = b.p16;
  va.t_max = b.t_max;
  va.t_sum = b.t_sum;
  va.t_arg = b.t_arg;
  va.n_tiles = b.n_tiles;
  va.dpart = b.dpart;
  va.n_dch = b.n_dch;
  va.dchunk = kDChunk;
  va.lse_q = b.lse_q;
  va.opart = b.opart;
  va.n_och = b.n_och;
  va.ochunk = kOChunk;
  va.argmax = out->argmax;
  va.accept_len = out->accept_len;
  va.bonus = out->bonus;
  va.last_row = out->last_row;
  va.row_max = out->row_max;
  va.row_lse = out->row_lse;
  va.overlap = out->overlap;
  va.survival = out->survival;
  va.surv_sum = out->surv_sum;
  return va;
}

// Device buffers of the fp32 path of one run.
struct F32Bufs {
  float *q_rot, *k_rot, *o_act, *h_part, *hn;
  float *t_max, *t_sum;   // the LM head's tile statistics
  int32_t *t_arg;
};

// fp32 models: RoPE, drafter statistics, attention, W_o, final norm, and the
// LM head with its tile statistics, as plain fp32 kernels.  `begin(name)` /
// `end()` bracket each stage (profiling events, or nothing).
template <class Begin, class End>
void enqueue_f32(const sv::Dims &dm, const sv_config &cfg, const char *m, const sv::MetaLayout &lay, const F32Bufs &b,
                 const void *w_o, const void *w_lm, const sv_inputs *in, const sv::VocabArgs &va, hipStream_t stream,
                 Begin &&begin, End &&end) {
  const int n = va.n, Hq = dm.Hq, Hkv = dm.Hkv, D = dm.d, H = dm.hidden, V = dm.vocab;
  begin("rope");
  sv::launch_rope_f32(static_cast<const float *>(in->q_rows), static_cast<const float *>(in->k_rows), b.q_rot,
                      b.k_rot, reinterpret_cast<const int32_t *>(m + lay.row_pos), n, Hq, Hkv, D,
                      double(cfg.rope_base), stream);
  end();
  begin("drafter_stats");
  sv::launch_drafter_partial(va, stream);
  end();
  sv::AttnF32Args af{};
  af.kv_k = static_cast<const float *>(in->kv_k);
  af.kv_v = static_cast<const float *>(in->kv_v);
  af.k_rot = b.k_rot;
  af.v_rows = static_cast<const float *>(in->v_rows);
  af.q_rot = b.q_rot;
  af.row_tree = reinterpret_cast<const int32_t *>(m + lay.row_tree);
  af.tree_start = reinterpret_cast<const int32_t *>(m + lay.tree_start);
  af.tree_rows = reinterpret_cast<const int32_t *>(m + lay.tree_rows);
  af.tree_kv_len = reinterpret_cast<const int32_t *>(m + lay.tree_kv_len);
  af.tree_kv_off = reinterpret_cast<const int64_t *>(m + lay.tree_kv_off);
  af.row_anc = reinterpret_cast<const uint64_t *>(m + lay.row_anc);
  af.out = b.o_act;
  af.Hq = Hq;
  af.Hkv = Hkv;
  af.D = D;
  begin("attention");
  sv::launch_attn_f32(af, n, stream);
  end();
  begin("w_o");
  sv::launch_gemm_f32(b.o_act, n, static_cast<const float *>(w_o), H, Hq * D, b.h_part, stream);
  end();
  begin("final_norm");
  sv::launch_norm(b.h_part, 1, 0, n, H, cfg.norm_eps, sv::ACT_F32, b.hn, 0, nullptr, stream);
  end();
  begin("lm_head");
  sv::launch_gemm_f32(b.hn, n, static_cast<const float *>(w_lm), V, H, va.logits, stream);
  sv::launch_stats_from_logits(va.logits, n, V, 256, b.t_max, b.t_sum, b.t_arg, va.n_tiles, stream);
  end();
}

// After the LM head: row statistics, overlaps, acceptance, and in T = 1 mode
// the stochastic walk and the bonus draw.
template <class Begin, class End>
void enqueue_tail(const sv::VocabArgs &va, const sv_inputs *in, const char *m, const sv::MetaLayout &lay,
                  int32_t *rej_child, float *rpart, hipStream_t stream, Begin &&begin, End &&end) {
  if (va.n <= 64) {
    // few rows: few tile records per row, so the overlap workgroups merge
    // their own logsumexps and the two passes share one launch; in small
    // launches the workgroup that completes a tree runs its acceptance walk
    const bool fused = sv::combine_overlap_accepts(va);
    begin(fused ? "combine_overlap_accept" : "combine_overlap");
    sv::launch_combine_overlap(va, stream);
    end();
    if (!fused) {
      begin("accept");
      sv::launch_accept(va, stream);
      end();
    }
  } else {
    begin("row_combine");
    sv::launch_row_combine(va, stream);
    end();
    begin("overlap");
    sv::launch_overlap_partial(va, stream);
    end();
    begin("accept");
    sv::launch_accept(va, stream);
    end();
  }
  if (in->mode == SV_MODE_SAMPLE) {
    sv::SampleArgs sa{};
    sa.row_child = reinterpret_cast<const int32_t *>(m + lay.row_child);
    sa.u_accept = in->u_accept;
    sa.u_bonus = in->u_bonus;
    sa.rej_child = rej_child;
    sa.rpart = rpart;
    begin("sample");
    sv::launch_sample(va, sa, stream);
    end();
  }
}

// Validation of one run's arguments and its plan (shared by spec_verify_run
// and spec_verify_run_static): nothing may be enqueued before this passes.
sv_status check_run(const sv::Dims &dm, const sv_inputs *in, const sv_outputs *out, int64_t slot_cap,
                    int target_items, int n_och, sv::Plan *plan, sv::MetaLayout *lay) {
  sv::HostInputs hi{in->n_rows, in->n_roots, in->parent, in->pos, in->root_kv_off, in->root_kv_len, in->kv_tokens};
  std::string err;
  const int pc = sv::build_plan(dm, hi, slot_cap, target_items, plan, &err);
  if (pc != sv::P_OK) return fail(sv_status(pc), err);
  if (!in->q_rows || !in->k_rows || !in->v_rows || !in->draft_ids)
    return fail(SV_ERR_INVALID_ARG, "q_rows, k_rows, v_rows and draft_ids must be non-null device pointers");
  if (plan->n_draft > 0 && !in->drafter_logits)
    return fail(SV_ERR_INVALID_ARG, "drafter_logits must be non-null when the block has draft rows");
  if (in->mode != SV_MODE_GREEDY && in->mode != SV_MODE_SAMPLE)
    return fail(SV_ERR_INVALID_ARG, "mode must be SV_MODE_GREEDY or SV_MODE_SAMPLE");
  if (in->mode == SV_MODE_SAMPLE) {
    if (!in->u_accept || !in->u_bonus) return fail(SV_ERR_INVALID_ARG, "SV_MODE_SAMPLE needs u_accept and u_bonus");
    if (!plan->chains_only)
      return fail(SV_ERR_UNSUPPORTED, "SV_MODE_SAMPLE takes chains: a row has more than one child");
    if (n_och > 1024) return fail(SV_ERR_UNSUPPORTED, "SV_MODE_SAMPLE supports vocabularies up to 8388608 tokens");
  }
  if (in->kv_tokens > 0 && (!in->kv_k || !in->kv_v))
    return fail(SV_ERR_INVALID_ARG, "kv_k and kv_v must be non-null when kv_tokens > 0");
  if (!out->accept_len || !out->bonus || !out->last_row || !out->surv_sum || !out->argmax || !out->row_max ||
      !out->row_lse || !out->overlap || !out->survival)
    return fail(SV_ERR_INVALID_ARG, "every output except logits must be a non-null device pointer");
  const bool samp = in->mode == SV_MODE_SAMPLE;
  const sv::RunPointers rp{{in->kv_tokens > 0 ? in->kv_k : nullptr, in->kv_tokens > 0 ? in->kv_v : nullptr,
                            in->q_rows, in->k_rows, in->v_rows, plan->n_draft > 0 ? in->drafter_logits : nullptr,
                            out->logits},
                           {in->draft_ids, samp ? in->u_accept : nullptr, samp ? in->u_bonus : nullptr,
                            out->accept_len, out->bonus, out->last_row, out->surv_sum, out->argmax, out->row_max,
                            out->row_lse, out->overlap, out->survival}};
  const int ac = sv::check_alignment(rp, &err);
  if (ac != sv::P_OK) return fail(sv_status(ac), err);
  *lay = sv::meta_layout(plan->n, plan->R, plan->n_draft, int(plan->items.size()), int(plan->runs.size()),
                         plan->R * dm.Hkv * plan->qg_max);
  return SV_OK;
}

}  // namespace


// ----------------------------------------------------------------------------
// spec_verify_run_static: a verify step of an fp32 model without a handle and
// without any allocation.  Every per-run buffer lives in `scratch`, one
// file-scope device array (each device the library runs on holds its own
// copy, at its own address, until the process ends); its device address is
// taken once per device with hipGetSymbolAddress, and only that address is
// ever given to kernels or copies.  The plan reaches the device as kernel
// arguments, kStaticChunkWords words per launch, so no host or pinned staging
// buffer has to outlive the call.
// ----------------------------------------------------------------------------

namespace {

constexpr size_t kStaticScratchBytes = size_t(8) << 20;
constexpr int kStaticMaxDevices = 64;
constexpr int kStaticChunkWords = 880;   // 3520 bytes of plan per launch (kernel arguments well under 4 KB)

std::mutex g_scratch_mu;
void *g_scratch_ptr[kStaticMaxDevices] = {};

}  // namespace

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

struct PlanChunk {
  uint32_t first, words;
  uint32_t w[kStaticChunkWords];
};

__global__ __launch_bounds__(256) void plan_chunk_kernel(PlanChunk c, uint32_t *dst) {
  for (uint32_t i = threadIdx.x; i < c.words; i += 256) dst[c.first + i] = c.w[i];
}

// The device address of `scratch` on device `dev` (the current device).
sv_status static_scratch(int dev, unsigned char **out) {
  if (dev < 0 || dev >= kStaticMaxDevices) return fail(SV_ERR_UNSUPPORTED, "device index beyond 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return hip_fail("hipGetSymbolAddress(scratch)", e);
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = static_cast<unsigned char *>(g_scratch_ptr[dev]);
  return SV_OK;
}

// Carves `scratch` into the run's buffers, 256-byte aligned, in order.
struct Carver {
  unsigned char *base;
  size_t used = 0;
  template <class T>
  T *take(size_t bytes) {
    T *p = reinterpret_cast<T *>(base + used);
    used += (std::max<size_t>(bytes, 1) + 255) / 256 * 256;
    return p;
  }
};

}  // namespace

extern "C" {

const char *spec_verify_last_error(void) { return g_err.c_str(); }

}  // extern "C"

namespace {

// Byte offsets of the parts of a prepared-weights buffer (spec_verify_weight_bytes).
struct PreparedLayout {
  size_t o16, o_blk, lm_blk, bad, total;
};

PreparedLayout prepared_layout(const sv::Dims &dm) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  const int64_t H = dm.hidden, K = int64_t(dm.Hq) * dm.d, V = dm.vocab;
  PreparedLayout L{};
  size_t o = 0;
  L.o16 = o;
  o = al(o + size_t(H * K * 2));
  L.o_blk = o;
  o = al(o + size_t(sv::blocked_elems(H, K) * 2));
  L.lm_blk = o;
  o = al(o + size_t(sv::blocked_elems(V, H) * 2));
  L.bad = o;
  L.total = o + 256;
  return L;
}

// The checks every prepared-weights call shares: dimensions, and a bf16
// model whose weights the library converts to fp16 (not FP8).
sv_status check_prepared_cfg(const sv_config *cfg, sv::Dims *dm) {
  if (!cfg) return fail(SV_ERR_INVALID_ARG, "cfg must be non-null");
  *dm = sv::Dims{cfg->n_q_heads, cfg->n_kv_heads, cfg->head_dim, cfg->hidden,        cfg->vocab,
                 cfg->dtype,     cfg->max_rows,   cfg->max_roots, cfg->max_tree_rows, cfg->max_pos,
                 cfg->weight_format};
  std::string err;
  const int pc = sv::check_dims(*dm, &err);
  if (pc != sv::P_OK) return fail(sv_status(pc), err);
  if (dm->dtype != SV_BF16 || dm->weight_format != SV_WEIGHTS_NATIVE)
    return fail(SV_ERR_UNSUPPORTED, "prepared weights are for bf16 models with the native (fp16) weight format");
  return SV_OK;
}

sv_status create_impl(const sv_config *cfg, const void *w_o, const void *w_lm, const unsigned char *prepared,
                      sv_handle **out) {
  g_err.clear();
  if (!cfg || !out) return fail(SV_ERR_INVALID_ARG, "cfg and out must be non-null");
  *out = nullptr;
  if (!prepared && (!w_o || !w_lm)) return fail(SV_ERR_INVALID_ARG, "w_o and w_lm must be non-null device pointers");
  sv::Dims dm{cfg->n_q_heads, cfg->n_kv_heads, cfg->head_dim, cfg->hidden, cfg->vocab, cfg->dtype,
              cfg->max_rows,  cfg->max_roots,  cfg->max_tree_rows, cfg->max_pos, cfg->weight_format};
  std::string err;
  const int pc = sv::check_dims(dm, &err);
  if (pc != sv::P_OK) return fail(sv_status(pc), err);
  if (!(cfg->rope_base > 1.0f) || !std::isfinite(cfg->rope_base))
    return fail(SV_ERR_INVALID_ARG, "rope_base must be a finite value > 1");
  if (!(cfg->norm_eps >= 0.0f) || !std::isfinite(cfg->norm_eps))
    return fail(SV_ERR_INVALID_ARG, "norm_eps must be finite and >= 0");

  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("hipGetDevice", e);
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return hip_fail("hipGetDeviceProperties", e);
  if (std::strstr(prop.gcnArchName, "gfx950") == nullptr)
    return fail(SV_ERR_UNSUPPORTED, std::string("device ") + std::to_string(dev) + " is " + prop.gcnArchName +
                                        "; this library is built for gfx950 (MI355X) only");

  sv_handle *h = new sv_handle();
  h->cfg = *cfg;
  h->dm = dm;
  h->w_o = w_o;
  h->w_lm = w_lm;
  h->device = dev;
  h->n_cu = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
  h->target_items = 2 * h->n_cu;   // attention runs: one per resident four-wave workgroup
  h->elt = dm.dtype == SV_BF16 ? 2 : 4;

  const int64_t R = dm.max_rows, Hq = dm.Hq, Hkv = dm.Hkv, D = dm.d, H = dm.hidden, V = dm.vocab;
  const int64_t E = h->elt;
  h->slot_cap = sv::slot_capacity(dm);
  // W_o split-K partials: the largest splits x rows any run up to max_rows needs
  int64_t part_rows = R;
  for (int n = 1; n <= dm.max_rows; ++n) {
    int ks = 0;
    part_rows = std::max<int64_t>(part_rows, int64_t(sv::gemm_splits(n, int(H), int(Hq * D), h->n_cu, &ks)) * n);
  }
  h->h_part_floats = size_t(part_rows) * H;
  h->n_tiles_cap = int(ceil_div(V, 128));
  h->n_dch = int(ceil_div(V, kDChunk));
  h->n_och = int(ceil_div(V, kOChunk));
  h->meta_cap = sv::meta_capacity(dm, h->target_items);

  sv_status st = SV_OK;
  auto A = [&](auto **p, size_t bytes) {
    if (st == SV_OK) st = dev_alloc(h, p, bytes);
  };
  A(&h->d_meta, h->meta_cap);
  A(&h->q_rot, size_t(R * Hq * D * 4));       // bf16: hi + lo planes; fp32: one plane
  A(&h->k_rot, size_t(R * Hkv * D * 4));      // bf16: hi + lo planes; fp32: one plane
  if (dm.dtype == SV_BF16) {
    A(&h->part_o, size_t(h->slot_cap * D * 4));
    A(&h->part_ml, size_t(h->slot_cap * 2 * 4));
  }
  // attention output: fp16 hi + lo planes, blocked fp16 (rows padded to 256), or fp32
  // (hi plane, then the lo plane one blocked capacity further)
  A(&h->o_act, std::max<size_t>(size_t(R * Hq * D * 4), size_t(2 * sv::blocked_elems(R, Hq * D) * 2)));
  A(&h->h_part, h->h_part_floats * 4);
  // normalised rows: fp16 hi + lo planes (<= 64 rows) or the blocked fp16
  // layout of the tiled LM head (rows padded to 256) and a row-major fp16 lo
  // plane, one blocked capacity further in both cases
  A(&h->hn, std::max<size_t>(size_t(R * H * 4), size_t((sv::blocked_elems(R, H) + R * H) * 2)));
  A(&h->logits, size_t(R * V * 4));
  if (dm.dtype == SV_BF16 && V % 8 == 0) A(&h->p16, size_t(R * V * 2));
  A(&h->t_max, size_t(R * h->n_tiles_cap * 4));
  A(&h->t_sum, size_t(R * h->n_tiles_cap * 4));
  A(&h->t_arg, size_t(R * h->n_tiles_cap * 4));
  A(&h->dpart, size_t(R * h->n_dch * 8));
  A(&h->lse_q, size_t(R * 4));
  A(&h->opart, size_t(R * h->n_och * 4));
  A(&h->rej_child, size_t(dm.max_roots) * 4);
  A(&h->rpart, size_t(dm.max_roots) * h->n_och * 4);
  if (dm.dtype == SV_BF16 && prepared) {
    // borrowed fp16 weights (spec_verify_prepare_weights): nothing to copy
    const PreparedLayout L = prepared_layout(dm);
    h->w_o = prepared + L.o16;
    h->w_o_blk = reinterpret_cast<const uint16_t *>(prepared + L.o_blk);
    h->w_lm = prepared + L.lm_blk;
    if (st == SV_OK) {
      // padding rows of the blocked activations are read by the LM head:
      // start them at zero
      e = hipMemsetAsync(h->hn, 0, std::max<size_t>(size_t(R * H * 4), size_t((sv::blocked_elems(R, H) + R * H) * 2)),
                         nullptr);
      if (e == hipSuccess) e = hipDeviceSynchronize();
      if (e != hipSuccess) {
        release(h);
        return hip_fail("hipMemsetAsync", e);
      }
    }
  } else if (dm.dtype == SV_BF16) {
    // the projections run on fp16 MFMA: keep fp16 copies of the weights
    // (W_o row-major, W_lm in the blocked layout)
    uint16_t *wo16 = nullptr, *wlm16 = nullptr, *wo_blk = nullptr;
    const bool fp8 = dm.weight_format == SV_WEIGHTS_FP8;
    const bool tiled = dm.max_rows > 64;
    A(&wo16, size_t(H * Hq * D * 2));
    if (tiled) A(&wo_blk, size_t(sv::blocked_elems(H, Hq * D) * 2));
    if (fp8) {
      A(&h->w_lm8, size_t(sv::blocked_elems(V, H)));
      A(&h->w_scale, size_t(ceil_div(V, 256) * 256 * 4));
      A(&h->a_scale, size_t(R * 4));
    } else {
      A(&wlm16, size_t(sv::blocked_elems(V, H) * 2));
    }
    A(&h->d_bad, 4);
    if (st == SV_OK) {
      e = hipMemsetAsync(h->d_bad, 0, 4, nullptr);
      // padding rows of the blocked activations are read by the LM head:
      // start them at zero
      if (e == hipSuccess)
        e = hipMemsetAsync(h->hn, 0, std::max<size_t>(size_t(R * H * 4), size_t((sv::blocked_elems(R, H) + R * H) * 2)),
                           nullptr);
      if (e == hipSuccess) {
        sv::launch_bf16_to_f16(static_cast<const uint16_t *>(w_o), wo16, H * Hq * D, h->d_bad, nullptr);
        if (tiled)
          sv::launch_bf16_to_f16_blocked(static_cast<const uint16_t *>(w_o), wo_blk, int(H), int(Hq * D), h->d_bad,
                                         nullptr);
        if (fp8)
          sv::launch_quant_fp8_blocked(static_cast<const uint16_t *>(w_lm), h->w_lm8, h->w_scale, int(V), int(H),
                                       h->d_bad, nullptr);
        else
          sv::launch_bf16_to_f16_blocked(static_cast<const uint16_t *>(w_lm), wlm16, int(V), int(H), h->d_bad,
                                         nullptr);
        e = hipGetLastError();
      }
      int32_t bad = 0;
      if (e == hipSuccess) e = hipMemcpy(&bad, h->d_bad, 4, hipMemcpyDeviceToHost);
      if (e != hipSuccess) {
        release(h);
        return hip_fail("weight conversion", e);
      }
      if (bad != 0) {
        release(h);
        return fail(SV_ERR_UNSUPPORTED,
                    std::to_string(bad) + (fp8 ? " weight values are not finite, or W_o values exceed the fp16 range"
                                               : " weight values exceed the fp16 range (|w| > 65504) or are not finite"));
      }
      h->w_o = wo16;
      h->w_o_blk = wo_blk;
      h->w_lm = wlm16;
    }
  }
  if (st != SV_OK) {
    release(h);
    return st;
  }
  for (int i = 0; i < kRing; ++i) {
    e = hipHostMalloc(reinterpret_cast<void **>(&h->h_meta[i]), h->meta_cap, hipHostMallocDefault);
    if (e != hipSuccess) {
      release(h);
      return fail(SV_ERR_OOM, std::string("hipHostMalloc: ") + hipGetErrorString(e));
    }
    e = hipEventCreateWithFlags(&h->meta_ev[i], hipEventDisableTiming);
    if (e != hipSuccess) {
      release(h);
      return hip_fail("hipEventCreate", e);
    }
  }
  e = hipEventCreateWithFlags(&h->done, hipEventDisableTiming);
  if (e != hipSuccess) {
    release(h);
    return hip_fail("hipEventCreate", e);
  }
  *out = h;
  return SV_OK;
}

}  // namespace

extern "C" {

sv_status spec_verify_create(const sv_config *cfg, const void *w_o, const void *w_lm, sv_handle **out) {
  return create_impl(cfg, w_o, w_lm, nullptr, out);
}

sv_status spec_verify_weight_bytes(const sv_config *cfg, size_t *bytes) {
  g_err.clear();
  if (!bytes) return fail(SV_ERR_INVALID_ARG, "bytes must be non-null");
  *bytes = 0;
  sv::Dims dm{};
  const sv_status st = check_prepared_cfg(cfg, &dm);
  if (st != SV_OK) return st;
  *bytes = prepared_layout(dm).total;
  return SV_OK;
}

sv_status spec_verify_prepare_weights(const sv_config *cfg, const void *w_o, const void *w_lm, void *dst,
                                      void *stream_v) {
  g_err.clear();
  sv::Dims dm{};
  const sv_status st = check_prepared_cfg(cfg, &dm);
  if (st != SV_OK) return st;
  if (!w_o || !w_lm || !dst) return fail(SV_ERR_INVALID_ARG, "w_o, w_lm and dst must be non-null device pointers");
  if (reinterpret_cast<uintptr_t>(dst) % 256 != 0) return fail(SV_ERR_INVALID_ARG, "dst must be 256-byte aligned");
  const PreparedLayout L = prepared_layout(dm);
  const hipStream_t stream = static_cast<hipStream_t>(stream_v);
  unsigned char *d = static_cast<unsigned char *>(dst);
  int32_t *bad = reinterpret_cast<int32_t *>(d + L.bad);
  const int64_t H = dm.hidden, K = int64_t(dm.Hq) * dm.d;
  hipError_t e = hipMemsetAsync(bad, 0, 4, stream);
  if (e != hipSuccess) return hip_fail("hipMemsetAsync", e);
  sv::launch_bf16_to_f16(static_cast<const uint16_t *>(w_o), reinterpret_cast<uint16_t *>(d + L.o16), H * K, bad,
                         stream);
  sv::launch_bf16_to_f16_blocked(static_cast<const uint16_t *>(w_o), reinterpret_cast<uint16_t *>(d + L.o_blk),
                                 int(H), int(K), bad, stream);
  sv::launch_bf16_to_f16_blocked(static_cast<const uint16_t *>(w_lm), reinterpret_cast<uint16_t *>(d + L.lm_blk),
                                 int(dm.vocab), int(H), bad, stream);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail("weight conversion", e);
  int32_t n_bad = 0;
  e = hipMemcpyAsync(&n_bad, bad, 4, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail("weight conversion", e);
  if (n_bad != 0)
    return fail(SV_ERR_UNSUPPORTED,
                std::to_string(n_bad) + " weight values exceed the fp16 range (|w| > 65504) or are not finite");
  return SV_OK;
}

sv_status spec_verify_create_prepared(const sv_config *cfg, const void *prepared, sv_handle **out) {
  g_err.clear();
  if (out) *out = nullptr;
  sv::Dims dm{};
  const sv_status st = check_prepared_cfg(cfg, &dm);
  if (st != SV_OK) return st;
  if (!prepared) return fail(SV_ERR_INVALID_ARG, "prepared must be a non-null device pointer");
  if (reinterpret_cast<uintptr_t>(prepared) % 256 != 0)
    return fail(SV_ERR_INVALID_ARG, "prepared must be 256-byte aligned");
  return create_impl(cfg, nullptr, nullptr, static_cast<const unsigned char *>(prepared), out);
}

sv_status spec_verify_destroy(sv_handle *h) {
  g_err.clear();
  if (!h) return SV_OK;
  sv_status st = SV_OK;
  if (h->ran) {
    const hipError_t e = hipEventSynchronize(h->done);
    if (e != hipSuccess) st = hip_fail("hipEventSynchronize", e);
  }
  release(h);
  return st;
}

static void drop_stages(sv_handle *h) {
  for (auto &s : h->stages) {
    (void)hipEventDestroy(s.a);
    (void)hipEventDestroy(s.b);
  }
  h->stages.clear();
}

sv_status spec_verify_profile(sv_handle *h, int32_t on) {  // on: profiling mode
  g_err.clear();
  if (!h) return fail(SV_ERR_INVALID_ARG, "null handle");
  if (h->ran) {
    const hipError_t e = hipEventSynchronize(h->done);
    if (e != hipSuccess) return hip_fail("hipEventSynchronize", e);
  }
  if (on < 0 || on > 2) return fail(SV_ERR_INVALID_ARG, "profile mode must be 0, 1 or 2");
  drop_stages(h);
  h->profile = on;
  return SV_OK;
}

int32_t spec_verify_stage_times(sv_handle *h, const char **names, float *ms, int32_t cap) {
  g_err.clear();
  if (!h) return fail(SV_ERR_INVALID_ARG, "null handle");
  if (h->stages.empty()) return 0;
  hipError_t e = hipEventSynchronize(h->stages.back().b);
  if (e != hipSuccess) return hip_fail("hipEventSynchronize", e);
  // mean per stage name, in order of first appearance
  std::vector<const char *> order;
  std::vector<double> sum;
  std::vector<int> cnt;
  for (const auto &s : h->stages) {
    float t = 0.f;
    e = hipEventElapsedTime(&t, s.a, s.b);
    if (e != hipSuccess) return hip_fail("hipEventElapsedTime", e);
    size_t k = 0;
    while (k < order.size() && std::strcmp(order[k], s.name) != 0) ++k;
    if (k == order.size()) {
      order.push_back(s.name);
      sum.push_back(0.0);
      cnt.push_back(0);
    }
    sum[k] += t;
    cnt[k] += 1;
  }
  const int n = int(std::min<size_t>(order.size(), size_t(std::max(cap, 0))));
  for (int i = 0; i < n; ++i) {
    if (names) names[i] = order[i];
    if (ms) ms[i] = float(sum[i] / cnt[i]);
  }
  return int32_t(order.size());
}

sv_status spec_verify_run(sv_handle *h, const sv_inputs *in, const sv_outputs *out, void *stream_v) {
  g_err.clear();
  if (!h || !in || !out) return fail(SV_ERR_INVALID_ARG, "handle, inputs and outputs must be non-null");
  const sv::Dims &dm = h->dm;
  const hipStream_t stream = static_cast<hipStream_t>(stream_v);

  // ---- host-side validation and plan (nothing is enqueued before this passes)
  sv::Plan plan;
  sv::MetaLayout lay{};
  {
    const sv_status vs = check_run(dm, in, out, h->slot_cap, h->target_items, h->n_och, &plan, &lay);
    if (vs != SV_OK) return vs;
  }
  if (lay.total > h->meta_cap) return fail(SV_ERR_CAPACITY, "metadata exceeds the handle's staging capacity");

  const int n = plan.n;
  const int64_t V = dm.vocab, H = dm.hidden, D = dm.d, Hq = dm.Hq, Hkv = dm.Hkv;
  const bool bf16 = dm.dtype == SV_BF16;

  size_t step_stage = 0;
  if (h->profile == 1) {
    Stage s{"step", nullptr, nullptr};
    (void)hipEventCreate(&s.a);
    (void)hipEventCreate(&s.b);
    h->stages.push_back(s);
    step_stage = h->stages.size() - 1;
  }
  // ---- metadata: pinned staging slot -> one async copy
  const int slot = h->ring;
  h->ring = (h->ring + 1) % kRing;
  hipError_t e;
  if (h->meta_used[slot]) {
    e = hipEventSynchronize(h->meta_ev[slot]);   // the copy issued kRing runs ago
    if (e != hipSuccess) return hip_fail("hipEventSynchronize", e);
  }
  sv::MetaLayout lay2;
  sv::pack_plan(plan, dm.Hkv, h->h_meta[slot], &lay2);
  if (h->profile == 1) (void)hipEventRecord(h->stages[step_stage].a, stream);
  e = hipMemcpyAsync(h->d_meta, h->h_meta[slot], lay.total, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return hip_fail("hipMemcpyAsync", e);
  e = hipEventRecord(h->meta_ev[slot], stream);
  if (e != hipSuccess) return hip_fail("hipEventRecord", e);
  h->meta_used[slot] = true;

  const char *m = h->d_meta;
  const int32_t *row_pos = reinterpret_cast<const int32_t *>(m + lay.row_pos);
  const int32_t *row_pack = reinterpret_cast<const int32_t *>(m + lay.row_pack);
  const int32_t *row_plocal = reinterpret_cast<const int32_t *>(m + lay.row_plocal);
  const int32_t *row_klen = reinterpret_cast<const int32_t *>(m + lay.row_klen);
  const uint64_t *row_panc = reinterpret_cast<const uint64_t *>(m + lay.row_panc);
  const sv::AttnItem *items = reinterpret_cast<const sv::AttnItem *>(m + lay.items);
  const sv::AttnRun *runs = reinterpret_cast<const sv::AttnRun *>(m + lay.runs);
  const sv::AttnGroup *groups = reinterpret_cast<const sv::AttnGroup *>(m + lay.groups);

  // ---- stage bookkeeping for profiling (events on the run's stream)
  bool recording = false;
  auto begin = [&](const char *name) {
    recording = h->profile == 1 || (h->profile == 2 && std::strcmp(name, "lm_head") == 0);
    if (!recording) return;
    Stage s{name, nullptr, nullptr};
    (void)hipEventCreate(&s.a);
    (void)hipEventCreate(&s.b);
    (void)hipEventRecord(s.a, stream);
    h->stages.push_back(s);
  };
  auto end = [&]() {
    if (!recording) return;
    (void)hipEventRecord(h->stages.back().b, stream);
    recording = false;
  };

  float *logits = out->logits ? out->logits : h->logits;
  const bool fp8 = dm.weight_format == SV_WEIGHTS_FP8;
  const int tile_w = bf16 && !fp8 ? sv::lm_tile_width(n, int(V), h->n_cu) : 256;
  const int n_tiles = int(ceil_div(V, tile_w));

  // Without a caller logits buffer, the LM head stores each tile's
  // probabilities relative to the tile maximum in fp16 instead of fp32
  // logits: half the bytes for their readers (the overlap pass, and in T = 1
  // mode the accept tests and the bonus draw), and half the bytes written
  // while the weights stream in (every LM head launch, fp16 or FP8).
  const bool use_p16 = bf16 && !out->logits && h->p16 != nullptr;
  sv::VocabArgs va = vocab_args(plan, m, lay, int(V), bf16, in, out,
                                VocabBufs{logits, use_p16 ? h->p16 : nullptr, h->t_max, h->t_sum, h->t_arg,
                                          n_tiles, h->dpart, h->n_dch, h->lse_q, h->opart, h->n_och});
  va.tile_shift = tile_w == 128 ? 7 : 8;

  int k_split = 0;
  const int splits = bf16 ? sv::gemm_splits(n, int(H), int(Hq * D), h->n_cu, &k_split) : 1;
  // activation format of the projections: fp16 hi + lo planes for the
  // skinny launch, blocked fp16 for the tiled one (e4m3 for the FP8 LM head)
  const int lm_act_mode = fp8 ? sv::ACT_FP8_BLOCKED : n <= 64 ? sv::ACT_SPLIT : sv::ACT_F16_BLOCKED;
  const int64_t q_lo = int64_t(dm.max_rows) * Hq * D;   // lo planes start one capacity further
  const int64_t k_lo = int64_t(dm.max_rows) * Hkv * D;
  const int64_t o_lo = sv::blocked_elems(dm.max_rows, Hq * D);
  const int64_t h_lo = sv::blocked_elems(dm.max_rows, H);
  if (bf16 && !fp8 && n > 64) {
    // the tiled LM head's plain fp16 activations: its high-probability
    // logits are recomputed from the hi + lo pair with the row statistics
    va.rf_w = static_cast<const uint16_t *>(h->w_lm);
    va.rf_hi = static_cast<const uint16_t *>(h->hn);
    va.rf_lo = va.rf_hi + h_lo;
    va.rf_K = int(H);
  }

  if (bf16) {
    sv::RopeArgs ra{};
    ra.q = static_cast<const uint16_t *>(in->q_rows);
    ra.k = static_cast<const uint16_t *>(in->k_rows);
    ra.q_out = static_cast<uint16_t *>(h->q_rot);
    ra.k_out = static_cast<uint16_t *>(h->k_rot);
    ra.row_pos = row_pos;
    ra.Hq = int(Hq);
    ra.Hkv = int(Hkv);
    ra.D = int(D);
    ra.base = double(h->cfg.rope_base);
    ra.q_lo_off = q_lo;
    ra.k_lo_off = k_lo;
    ra.n = n;
    // workgroups per row: about 256 in all (each builds its row's table once),
    // at most one per 256 (head, pair) items; above 256 rows one per row (448
    // rows: 896 -> 448 workgroups, the RoPE + drafter stage 31.6 -> 29.3 us)
    ra.ry = int(std::max<int64_t>(1, std::min<int64_t>(ceil_div(int64_t(Hq + Hkv) * (D / 2), 256),
                                                       ceil_div(256, int64_t(n)))));
    begin("rope_drafter_stats");
    sv::launch_rope_drafter_bf16(ra, va, stream);
    end();
    sv::AttnArgs aa{};
    aa.kv_k = static_cast<const uint16_t *>(in->kv_k);
    aa.kv_v = static_cast<const uint16_t *>(in->kv_v);
    aa.k_rot = static_cast<const uint16_t *>(h->k_rot);
    aa.v_rows = static_cast<const uint16_t *>(in->v_rows);
    aa.q_rot = static_cast<const uint16_t *>(h->q_rot);
    aa.q_lo_off = q_lo;
    aa.items = items;
    aa.runs = runs;
    aa.row_panc = row_panc;
    aa.row_klen = row_klen;
    aa.part_o = h->part_o;
    aa.part_ml = h->part_ml;
    aa.Hq = int(Hq);
    aa.Hkv = int(Hkv);
    aa.G = int(Hq / Hkv);
    aa.scale_log2 = float(1.4426950408889634 / std::sqrt(double(D)));
    // Partial o records with the non-temporal hint when the K/V tiles streamed
    // exceed the 256 MB last-level cache: the record stores then leave the
    // KV stream alone (32 chains over 1.28 GB of K/V tiles: attention
    // 230 -> 222 us, merge 21 -> 26 us, which reads them from HBM instead).
    // With less KV the merge's cached reads win (the 17-row, 8192-prefix
    // chain: attention -1, merge +4 us).
    int64_t kv_tile_bytes = 0;
    for (const auto &it : plan.items) kv_tile_bytes += int64_t(it.k1 - it.k0) * D * 4;
    aa.nt_part = kv_tile_bytes > (int64_t(256) << 20) ? 1 : 0;
    int max_nq = 1;
    for (const auto &it : plan.items) max_nq = std::max(max_nq, int(it.nq));
    begin("attention");
    sv::launch_attn_mfma(aa, int(plan.runs.size()), int(D), int(ceil_div(max_nq, 16)), stream);
    end();
    sv::MergeArgs ma{};
    ma.part_o = h->part_o;
    ma.part_ml = h->part_ml;
    ma.groups = groups;
    ma.row_tree = row_pack;
    ma.row_local = row_plocal;
    ma.Hq = int(Hq);
    ma.Hkv = int(Hkv);
    ma.qg_max = plan.qg_max;
    ma.mode = n <= 64 ? sv::ACT_SPLIT : sv::ACT_SPLIT_BLOCKED;
    ma.lo_off = o_lo;
    ma.out = static_cast<uint16_t *>(h->o_act);
    ma.row_anc = reinterpret_cast<const uint64_t *>(m + lay.row_anc);
    ma.row_tree_real = reinterpret_cast<const int32_t *>(m + lay.row_tree);
    ma.tree_start = reinterpret_cast<const int32_t *>(m + lay.tree_start);
    ma.q_rot = aa.q_rot;
    ma.k_rot = aa.k_rot;
    ma.v_rows = aa.v_rows;
    ma.q_lo_off = q_lo;
    ma.k_lo_off = k_lo;
    ma.scale_log2 = aa.scale_log2;
    begin("attn_merge");
    int n_groups_used = 0;
    for (const auto &gr : plan.groups) n_groups_used += gr.count > 0;
    sv::launch_attn_merge(ma, n, int(D), double(plan.items.size()) / std::max(n_groups_used, 1), stream);
    end();
    sv::GemmArgs g{};
    g.act = static_cast<const uint16_t *>(h->o_act);
    g.act_lo = g.act + o_lo;
    g.rows = n;
    g.W = static_cast<const uint16_t *>(n <= 64 ? h->w_o : h->w_o_blk);
    g.N = int(H);
    g.K = int(Hq * D);
    g.k_split = k_split;
    g.out = h->h_part;
    g.ldo = H;
    g.split_stride = int64_t(n) * H;
    begin("w_o");
    sv::launch_gemm_bf16(g, false, splits, stream, n > 64, n > 64);
    end();
    begin("final_norm");
    sv::launch_norm(h->h_part, splits, int64_t(n) * H, n, int(H), h->cfg.norm_eps, lm_act_mode, h->hn, h_lo,
                    h->a_scale, stream);
    end();
    sv::GemmArgs l{};
    l.act = static_cast<const uint16_t *>(h->hn);
    l.act_lo = l.act + h_lo;
    l.rows = n;
    l.W = static_cast<const uint16_t *>(h->w_lm);
    l.N = int(V);
    l.K = int(H);
    l.k_split = int(H);
    l.out = logits;
    l.ldo = V;
    l.split_stride = 0;
    l.t_max = h->t_max;
    l.t_sum = h->t_sum;
    l.t_arg = h->t_arg;
    l.n_tiles = n_tiles;
    l.p16 = use_p16 ? h->p16 : nullptr;
    l.lm_narrow = tile_w == 128 ? 1 : 0;
    begin("lm_head");
    if (fp8) {
      l.W8 = h->w_lm8;
      l.act8 = static_cast<const uint8_t *>(h->hn);
      l.w_scale = h->w_scale;
      l.a_scale = h->a_scale;
      sv::launch_gemm_fp8(l, stream);
    } else {
      sv::launch_gemm_bf16(l, true, 1, stream);
    }
    end();
  } else {
    enqueue_f32(dm, h->cfg, m, lay,
                F32Bufs{static_cast<float *>(h->q_rot), static_cast<float *>(h->k_rot), static_cast<float *>(h->o_act),
                        h->h_part, static_cast<float *>(h->hn), h->t_max, h->t_sum, h->t_arg},
                h->w_o, h->w_lm, in, va, stream, begin, end);
  }
  enqueue_tail(va, in, m, lay, h->rej_child, h->rpart, stream, begin, end);
  if (h->profile == 1) (void)hipEventRecord(h->stages[step_stage].b, stream);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail("kernel launch", e);
  e = hipEventRecord(h->done, stream);
  if (e != hipSuccess) return hip_fail("hipEventRecord", e);
  h->ran = true;
  {
    auto &L = h->last;
    L.valid = true;
    L.stream = stream_v;
    L.n = n;
    L.R = plan.R;
    L.kv_tokens = in->kv_tokens;
    L.v_rows = in->v_rows;
    L.parent.assign(in->parent, in->parent + n);
    L.pos.assign(in->pos, in->pos + n);
    L.kv_off = plan.tree_kv_off;
    L.kv_len = plan.tree_kv_len;
    L.depth.assign(plan.R, 0);
    std::vector<int32_t> dep(n, 0);
    for (int i = 0; i < n; ++i) {
      dep[i] = in->parent[i] < 0 ? 0 : dep[in->parent[i]] + 1;
      L.depth[plan.row_tree[i]] = std::max(L.depth[plan.row_tree[i]], dep[i]);
    }
    L.lay = lay;
  }
  return SV_OK;
}

sv_status spec_verify_schedule(int32_t n_req, const int32_t *n_cand, const int32_t *cand_parent,
                               const float *cand_conf, int32_t n_curve, const int32_t *curve_rows,
                               const float *curve_ms, int32_t max_rows, int32_t *selected,
                               double *expected_tokens, double *step_ms) {
  g_err.clear();
  std::string err;
  const int st = sv::schedule_budget(n_req, n_cand, cand_parent, cand_conf, n_curve, curve_rows, curve_ms, max_rows,
                                     selected, expected_tokens, step_ms, &err);
  if (st != sv::P_OK) return fail(sv_status(st), err);
  return SV_OK;
}

sv_status spec_verify_commit(sv_handle *h, const sv_inputs *in, const sv_outputs *out, void *kv_k, void *kv_v,
                             void *stream_v) {
  g_err.clear();
  if (!h || !in || !out) return fail(SV_ERR_INVALID_ARG, "handle, inputs and outputs must be non-null");
  const auto &L = h->last;
  if (!L.valid) return fail(SV_ERR_INVALID_ARG, "spec_verify_commit follows a spec_verify_run on the same handle");
  if (stream_v != L.stream)
    return fail(SV_ERR_INVALID_ARG, "spec_verify_commit must be enqueued on the stream of the run it commits");
  const int n = L.n, R = L.R;
  bool same = in->n_rows == n && in->n_roots == R && in->parent && in->pos && in->root_kv_off && in->root_kv_len &&
              in->kv_tokens == L.kv_tokens && in->v_rows == L.v_rows;
  if (same) same = std::equal(L.parent.begin(), L.parent.end(), in->parent) &&
                   std::equal(L.pos.begin(), L.pos.end(), in->pos) &&
                   std::equal(L.kv_off.begin(), L.kv_off.end(), in->root_kv_off) &&
                   std::equal(L.kv_len.begin(), L.kv_len.end(), in->root_kv_len);
  if (!same) return fail(SV_ERR_INVALID_ARG, "inputs differ from those of the handle's most recent run");
  if (!out->accept_len || !out->last_row)
    return fail(SV_ERR_INVALID_ARG, "accept_len and last_row must be the device outputs of that run");
  if (!kv_k || !kv_v) return fail(SV_ERR_INVALID_ARG, "kv_k and kv_v must be non-null");
  if ((reinterpret_cast<uintptr_t>(kv_k) | reinterpret_cast<uintptr_t>(kv_v) |
       reinterpret_cast<uintptr_t>(in->v_rows)) % 16 != 0)
    return fail(SV_ERR_INVALID_ARG, "kv_k, kv_v and v_rows must be 16-byte aligned");
  // write ranges: tree t may write [off + len, off + len + depth + 1); none
  // may leave the cache or meet another tree's prefix or write range
  struct Iv {
    int64_t a, b;
    int t;   // tree of a write range, -1 for a prefix
  };
  std::vector<Iv> iv;
  iv.reserve(2 * size_t(R));
  for (int t = 0; t < R; ++t) {
    const int64_t w0 = L.kv_off[t] + L.kv_len[t], w1 = w0 + L.depth[t] + 1;
    if (w1 > L.kv_tokens)
      return fail(SV_ERR_BAD_TREE, "tree " + std::to_string(t) + ": its accepted path may need cache entries up to " +
                                       std::to_string(w1) + " but kv_tokens is " + std::to_string(L.kv_tokens));
    if (L.kv_len[t] > 0) iv.push_back({L.kv_off[t], w0, -1});
    iv.push_back({w0, w1, t});
  }
  std::sort(iv.begin(), iv.end(), [](const Iv &x, const Iv &y) { return x.a < y.a || (x.a == y.a && x.b < y.b); });
  int64_t max_end = INT64_MIN;
  for (size_t i = 0; i < iv.size(); ++i) {
    if (iv[i].t >= 0 && (iv[i].a < max_end || (i + 1 < iv.size() && iv[i + 1].a < iv[i].b)))
      return fail(SV_ERR_BAD_TREE, "tree " + std::to_string(iv[i].t) +
                                       ": the cache entries after its prefix overlap another tree's prefix or path");
    max_end = std::max(max_end, iv[i].b);
  }

  const hipStream_t stream = static_cast<hipStream_t>(stream_v);
  const char *m = h->d_meta;
  sv::CommitArgs ca{};
  ca.row_parent = reinterpret_cast<const int32_t *>(m + L.lay.row_parent);
  ca.tree_start = reinterpret_cast<const int32_t *>(m + L.lay.tree_start);
  ca.tree_rows = reinterpret_cast<const int32_t *>(m + L.lay.tree_rows);
  ca.accept_len = out->accept_len;
  ca.last_row = out->last_row;
  ca.kv_off = reinterpret_cast<const int64_t *>(m + L.lay.tree_kv_off);
  ca.kv_len = reinterpret_cast<const int32_t *>(m + L.lay.tree_kv_len);
  ca.k_rot = static_cast<const uint8_t *>(h->k_rot);
  ca.v_rows = static_cast<const uint8_t *>(in->v_rows);
  ca.kv_k = static_cast<uint8_t *>(kv_k);
  ca.kv_v = static_cast<uint8_t *>(kv_v);
  ca.row_bytes = int(int64_t(h->dm.Hkv) * h->dm.d * h->elt);
  sv::launch_commit(ca, R, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail("kernel launch", e);
  e = hipEventRecord(h->done, stream);
  if (e != hipSuccess) return hip_fail("hipEventRecord", e);
  return SV_OK;
}

sv_status spec_verify_run_static(const sv_config *cfg, const void *w_o, const void *w_lm, const sv_inputs *in,
                                 const sv_outputs *out, void *stream_v) {
  g_err.clear();
  if (!cfg || !in || !out) return fail(SV_ERR_INVALID_ARG, "cfg, inputs and outputs must be non-null");
  if (!w_o || !w_lm) return fail(SV_ERR_INVALID_ARG, "w_o and w_lm must be non-null device pointers");
  const sv::Dims dm{cfg->n_q_heads, cfg->n_kv_heads, cfg->head_dim, cfg->hidden,        cfg->vocab,
                    cfg->dtype,     cfg->max_rows,   cfg->max_roots, cfg->max_tree_rows, cfg->max_pos,
                    cfg->weight_format};
  std::string err;
  const int pc = sv::check_dims(dm, &err);
  if (pc != sv::P_OK) return fail(sv_status(pc), err);
  if (dm.dtype != SV_F32 || dm.weight_format != SV_WEIGHTS_NATIVE)
    return fail(SV_ERR_UNSUPPORTED, "spec_verify_run_static takes fp32 models (weights used as given)");
  if (!(cfg->rope_base > 1.0f) || !std::isfinite(cfg->rope_base))
    return fail(SV_ERR_INVALID_ARG, "rope_base must be a finite value > 1");
  if (!(cfg->norm_eps >= 0.0f) || !std::isfinite(cfg->norm_eps))
    return fail(SV_ERR_INVALID_ARG, "norm_eps must be finite and >= 0");
  if ((reinterpret_cast<uintptr_t>(w_o) | reinterpret_cast<uintptr_t>(w_lm)) % 16 != 0)
    return fail(SV_ERR_INVALID_ARG, "w_o and w_lm must be 16-byte aligned");
  const int64_t V = dm.vocab, H = dm.hidden, D = dm.d, Hq = dm.Hq, Hkv = dm.Hkv;
  const int n_dch = int(ceil_div(V, kDChunk)), n_och = int(ceil_div(V, kOChunk)), n_tiles = int(ceil_div(V, 256));
  sv::Plan plan;
  sv::MetaLayout lay{};
  {
    const sv_status vs = check_run(dm, in, out, sv::slot_capacity(dm), 1, n_och, &plan, &lay);
    if (vs != SV_OK) return vs;
  }
  const int64_t n = plan.n, nd = plan.n_draft, R = plan.R;
  // the run's buffers, in the order they are carved from `scratch`
  const size_t need_meta = (lay.total + 255) / 256 * 256;
  const size_t f = 4;
  const size_t sizes[] = {need_meta,
                          size_t(n * Hq * D) * f,               // rotated queries
                          size_t(n * Hkv * D) * f,              // rotated row keys
                          size_t(n * Hq * D) * f,               // attention output
                          size_t(n * H) * f,                    // W_o output
                          size_t(n * H) * f,                    // normalised rows
                          out->logits ? 0 : size_t(n * V) * f,  // logits
                          size_t(n * n_tiles) * f,              // tile max
                          size_t(n * n_tiles) * f,              // tile sum
                          size_t(n * n_tiles) * f,              // tile argmax
                          size_t(nd * n_dch) * 8,               // drafter chunk records
                          size_t(nd) * f,                       // drafter logsumexp
                          size_t(nd * n_och) * f,               // overlap chunk sums
                          size_t(R) * f,                        // rejected child (T = 1)
                          size_t(R * n_och) * f};               // bonus chunk sums (T = 1)
  size_t total = 0;
  for (size_t b : sizes) total += (std::max<size_t>(b, 1) + 255) / 256 * 256;
  if (total > kStaticScratchBytes)
    return fail(SV_ERR_CAPACITY, "this run needs " + std::to_string(total) + " bytes of scratch; " +
                                     "spec_verify_run_static has " + std::to_string(kStaticScratchBytes));

  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("hipGetDevice", e);
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return hip_fail("hipGetDeviceProperties", e);
  if (std::strstr(prop.gcnArchName, "gfx950") == nullptr)
    return fail(SV_ERR_UNSUPPORTED, std::string("device ") + std::to_string(dev) + " is " + prop.gcnArchName +
                                        "; this library is built for gfx950 (MI355X) only");
  unsigned char *base = nullptr;
  {
    const sv_status ss = static_scratch(dev, &base);
    if (ss != SV_OK) return ss;
  }
  Carver cv{base};
  char *m = cv.take<char>(sizes[0]);
  F32Bufs fb{};
  fb.q_rot = cv.take<float>(sizes[1]);
  fb.k_rot = cv.take<float>(sizes[2]);
  fb.o_act = cv.take<float>(sizes[3]);
  fb.h_part = cv.take<float>(sizes[4]);
  fb.hn = cv.take<float>(sizes[5]);
  float *logits = out->logits ? out->logits : cv.take<float>(sizes[6]);
  fb.t_max = cv.take<float>(sizes[7]);
  fb.t_sum = cv.take<float>(sizes[8]);
  fb.t_arg = cv.take<int32_t>(sizes[9]);
  float2 *dpart = cv.take<float2>(sizes[10]);
  float *lse_q = cv.take<float>(sizes[11]);
  float *opart = cv.take<float>(sizes[12]);
  int32_t *rej_child = cv.take<int32_t>(sizes[13]);
  float *rpart = cv.take<float>(sizes[14]);

  // the plan: packed on the host, sent as kernel arguments
  const hipStream_t stream = static_cast<hipStream_t>(stream_v);
  std::vector<uint32_t> words((lay.total + 3) / 4, 0u);
  sv::MetaLayout lay2{};
  sv::pack_plan(plan, dm.Hkv, words.data(), &lay2);
  PlanChunk chunk;
  for (size_t first = 0; first < words.size(); first += kStaticChunkWords) {
    chunk.first = uint32_t(first);
    chunk.words = uint32_t(std::min<size_t>(kStaticChunkWords, words.size() - first));
    std::memcpy(chunk.w, words.data() + first, chunk.words * 4);
    hipLaunchKernelGGL(plan_chunk_kernel, dim3(1), dim3(256), 0, stream, chunk, reinterpret_cast<uint32_t *>(m));
  }
  sv::VocabArgs va = vocab_args(plan, m, lay, int(V), false, in, out,
                                VocabBufs{logits, nullptr, fb.t_max, fb.t_sum, fb.t_arg, n_tiles, dpart, n_dch, lse_q,
                                          opart, n_och});
  auto none = [](const char *) {};
  auto none_end = []() {};
  enqueue_f32(dm, *cfg, m, lay, fb, w_o, w_lm, in, va, stream, none, none_end);
  enqueue_tail(va, in, m, lay, rej_child, rpart, stream, none, none_end);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail("kernel launch", e);
  return SV_OK;
}

}  // extern "C"
