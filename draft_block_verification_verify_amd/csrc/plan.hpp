// Host-side planning of one verify step: argument and tree validation, per-row
// tree metadata and the attention work list.  Pure C++17, no HIP, so it can be
// compiled and tested on a machine without a GPU.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace sv {

// Query vectors of one attention query group: the (row, head-in-group) pairs
// of one tree for one KV head, at most kItemQ of them per group.
constexpr int kItemQ = 128;
constexpr int kMaxTreeRows = 64;   // ancestor masks are one uint64 per row
constexpr int kMaxSplits = 1024;   // most work items per query group

struct Dims {
  int32_t Hq, Hkv, d, hidden, vocab, dtype;
  int32_t max_rows, max_roots, max_tree_rows, max_pos;
  int32_t weight_format = 0;   // 0 native, 1 FP8 LM head (bf16 only)
};

// Keys per attention tile for head dimension d: one tile of K (or V) is
// 16 KB of bf16.
constexpr int attn_key_tile(int d) { return 8192 / d; }

// Virtual key sequence of a tree, in tiles of KT = attn_key_tile(d) keys:
// prefix tiles [0, ceil(len / KT)) hold prefix tokens 0..len-1 (the last tile
// padded), then ceil(T / KT) row tiles hold the tree's T rows in row order.
// A tile never mixes the prefix with the rows.
//
// Query group: query vectors [m0, m0+nq) of (tree, kv head g), where
// m = local_row * G + head_in_group.  The attention work is the sequence of
// all query groups' tiles, group after group; it is cut into runs of equal
// length, one workgroup each, so a run may end inside a group and the next
// run continue it.
//
// One attention work item: the part of one query group that one run covers,
// tiles [k0 / KT, k1 / KT) of the tree's sequence (k0, k1 in keys, multiples
// of KT).  It leaves one partial (max, sum, o) record per query vector from
// `slot` on.  The item also carries its tree's first row, row count, prefix
// length and prefix offset.
struct AttnItem {
  int32_t tree, g, m0, nq, k0, k1, slot, tree_start;
  int32_t tree_rows, kv_len;
  int64_t kv_off;
  int32_t kv_min, pad;   // the smallest prefix length among the item's queries
};
static_assert(sizeof(AttnItem) == 56, "AttnItem layout");

// One workgroup's run: items [first, first + count) in order, `tiles` tiles
// in all.
struct AttnRun {
  int32_t first, count, tiles, pad;
};
static_assert(sizeof(AttnRun) == 16, "AttnRun layout");

// One query group for the merge: its items [first, first + count) (in
// order), the partial slot of its first item's first query and its query
// count nq; item t's record for query mi sits at slot + t * nq + mi.
struct AttnGroup {
  int32_t first, count, slot, nq;
};
static_assert(sizeof(AttnGroup) == 16, "AttnGroup layout");

struct HostInputs {
  int32_t n_rows, n_roots;
  const int32_t *parent, *pos;
  const int64_t *root_kv_off;
  const int32_t *root_kv_len;
  int64_t kv_tokens;
};

struct Plan {
  int32_t n = 0, R = 0, n_draft = 0;
  // per row
  std::vector<int32_t> row_tree, row_local, row_pos, row_parent, row_draft;
  std::vector<uint64_t> row_anc;     // ancestor-or-self bits, tree-local
  std::vector<int32_t> row_child;    // the row's child, -1 if none (last one if several)
  bool chains_only = true;           // no row has more than one child
  // per draft row: its global row
  std::vector<int32_t> draft_row;
  // per tree
  std::vector<int32_t> tree_start, tree_rows, tree_kv_len;
  std::vector<int64_t> tree_kv_off;
  // attention packs: consecutive trees over one KV segment whose queries
  // share one query group per KV head, so that each prefix tile is read once
  // for all of them (a pack of one tree otherwise).  Per row: its pack, its
  // row within the pack, its own prefix length (the keys of the shared
  // segment it sees) and its ancestor-or-self bits relative to the pack's
  // first row.
  int32_t n_packs = 0;
  std::vector<int32_t> row_pack, row_plocal, row_klen;
  std::vector<uint64_t> row_panc;
  // attention
  std::vector<AttnItem> items;        // in query-group order (tree fields: the pack's)
  std::vector<AttnRun> runs;          // one per attention workgroup
  int32_t qg_max = 1;                 // query groups per (tree, g)
  std::vector<AttnGroup> groups;      // [R * Hkv * qg_max], indexed by pack
  int32_t chunk = 0;                  // keys per run (the last run shorter)
  int64_t slots = 0;                  // partial (m, l, o) records needed
};

// Validation status codes (same values as sv_status).
enum PlanStatus { P_OK = 0, P_INVALID = -1, P_BAD_TREE = -2, P_CAPACITY = -3, P_UNSUPPORTED = -4 };

// Check the model description and capacities.
int check_dims(const Dims &dm, std::string *err);

// Device buffers of one run.  The kernels move the large ones (`wide`: KV
// cache, row q/k/v, drafter logits, caller logits) with 16-byte vector
// accesses and the small per-row and per-tree arrays (`narrow`: draft ids,
// uniforms, the outputs) with 4-byte ones.  Null entries are not checked
// here.
struct RunPointers {
  static constexpr int kWide = 7, kNarrow = 12;
  const void *wide[kWide];
  const void *narrow[kNarrow];
};
extern const char *const kWideNames[RunPointers::kWide];
extern const char *const kNarrowNames[RunPointers::kNarrow];

// P_INVALID, naming the first buffer that is not 16-byte (wide) or 4-byte
// (narrow) aligned; P_OK otherwise.
int check_alignment(const RunPointers &p, std::string *err);

// Validate the host inputs of one run and build its plan.  `slot_cap` bounds
// plan->slots; the work split is coarsened until it fits.  `target_items`
// is the run (workgroup) count to aim for.
int build_plan(const Dims &dm, const HostInputs &in, int64_t slot_cap, int target_items,
               Plan *plan, std::string *err);

// Attention partial records that a handle reserves for the given shape.
int64_t slot_capacity(const Dims &dm);

// Byte layout of the device copy of a plan (offsets into one buffer).
struct MetaLayout {
  size_t row_tree, row_local, row_pos, row_parent, row_draft, row_anc, row_child, draft_row;
  size_t row_pack, row_plocal, row_klen, row_panc;
  size_t tree_start, tree_rows, tree_kv_len, tree_kv_off;
  size_t tree_done;   // per-tree completion counters, zero in every upload
  size_t items, runs, groups;
  size_t total;
};
MetaLayout meta_layout(int n, int R, int n_draft, int n_items, int n_runs, int n_groups);
// Upper bound of the meta buffer for a handle's capacities.
size_t meta_capacity(const Dims &dm, int target_items);
// Serialise the plan into `dst` (at least meta_layout(...).total bytes).
void pack_plan(const Plan &p, int Hkv, void *dst, MetaLayout *lay);

}  // namespace sv
