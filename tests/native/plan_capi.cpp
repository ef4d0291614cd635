// Test-only C entry to the host planner (plan.cpp), built with g++ on a
// machine without a GPU: validation status, error text, per-row ancestor
// masks, the attention work items and the workgroup runs.
#include <cstring>
#include <string>

#include "plan.hpp"

extern "C" int svp_plan(const int *dims, int n_rows, int n_roots, const int32_t *parent, const int32_t *pos,
                        const int64_t *off, const int32_t *len, int64_t kv_tokens, int64_t slot_cap,
                        int target_items, int64_t *stats, char *err, int err_cap, uint64_t *anc_out,
                        int32_t *items_out, int items_cap, int32_t *runs_out, int runs_cap) {
  sv::Dims dm{dims[0], dims[1], dims[2], dims[3], dims[4], dims[5], dims[6], dims[7], dims[8], dims[9]};
  std::string e;
  int st = sv::check_dims(dm, &e);
  sv::Plan p;
  if (st == sv::P_OK) {
    sv::HostInputs hi{n_rows, n_roots, parent, pos, off, len, kv_tokens};
    st = sv::build_plan(dm, hi, slot_cap, target_items, &p, &e);
  }
  if (err && err_cap > 0) {
    std::strncpy(err, e.c_str(), size_t(err_cap - 1));
    err[err_cap - 1] = 0;
  }
  if (st != sv::P_OK) return st;
  stats[0] = p.R;
  stats[1] = p.n_draft;
  stats[2] = int64_t(p.items.size());
  stats[3] = p.slots;
  stats[4] = p.chunk;
  stats[5] = p.qg_max;
  stats[6] = int64_t(sv::meta_layout(p.n, p.R, p.n_draft, int(p.items.size()), int(p.runs.size()),
                                          p.R * dm.Hkv * p.qg_max).total);
  stats[7] = int64_t(sv::meta_capacity(dm, target_items));
  for (int i = 0; i < p.n; ++i) anc_out[i] = p.row_anc[i];
  const int ni = int(p.items.size()) < items_cap ? int(p.items.size()) : items_cap;
  std::memcpy(items_out, p.items.data(), sizeof(sv::AttnItem) * size_t(ni));
  stats[8] = int64_t(p.runs.size());
  const int nr = int(p.runs.size()) < runs_cap ? int(p.runs.size()) : runs_cap;
  std::memcpy(runs_out, p.runs.data(), sizeof(sv::AttnRun) * size_t(nr));
  return 0;
}

// Per-row attention pack arrays of the same plan: pack index, row within the
// pack, prefix length, pack-relative ancestor bits; returns the pack count.
extern "C" int svp_packs(const int *dims, int n_rows, int n_roots, const int32_t *parent, const int32_t *pos,
                         const int64_t *off, const int32_t *len, int64_t kv_tokens, int32_t *row_pack,
                         int32_t *row_plocal, int32_t *row_klen, uint64_t *row_panc) {
  sv::Dims dm{dims[0], dims[1], dims[2], dims[3], dims[4], dims[5], dims[6], dims[7], dims[8], dims[9]};
  std::string e;
  if (sv::check_dims(dm, &e) != sv::P_OK) return -100;
  sv::Plan p;
  sv::HostInputs hi{n_rows, n_roots, parent, pos, off, len, kv_tokens};
  const int st = sv::build_plan(dm, hi, int64_t(1) << 20, 1024, &p, &e);
  if (st != sv::P_OK) return st;
  for (int i = 0; i < p.n; ++i) {
    row_pack[i] = p.row_pack[i];
    row_plocal[i] = p.row_plocal[i];
    row_klen[i] = p.row_klen[i];
    row_panc[i] = p.row_panc[i];
  }
  return p.n_packs;
}

// Alignment check of a run's device buffers (the check spec_verify_run makes
// before anything is enqueued): 7 wide and 12 narrow pointers, in the order
// of sv::RunPointers.
extern "C" int svp_check_alignment(const void *const *wide, const void *const *narrow, char *err, int err_cap) {
  sv::RunPointers p{};
  for (int i = 0; i < sv::RunPointers::kWide; ++i) p.wide[i] = wide[i];
  for (int i = 0; i < sv::RunPointers::kNarrow; ++i) p.narrow[i] = narrow[i];
  std::string e;
  const int st = sv::check_alignment(p, &e);
  if (err && err_cap > 0) {
    std::strncpy(err, e.c_str(), size_t(err_cap - 1));
    err[err_cap - 1] = 0;
  }
  return st;
}
