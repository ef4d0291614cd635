// Host-side planning of one verify step (see plan.hpp).
#include "plan.hpp"

#include <algorithm>
#include <cstring>
#include <sstream>

namespace sv {

namespace {

template <class... A>
std::string cat(A &&...a) {
  std::ostringstream s;
  (s << ... << a);
  return s.str();
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align16(size_t x) { return (x + 15) & ~size_t(15); }

}  // namespace

int check_dims(const Dims &dm, std::string *err) {
  if (dm.Hq < 1 || dm.Hkv < 1 || dm.Hq % dm.Hkv != 0) {
    *err = cat("n_q_heads (", dm.Hq, ") must be a positive multiple of n_kv_heads (", dm.Hkv, ")");
    return P_INVALID;
  }
  if (dm.d != 64 && dm.d != 128 && dm.d != 256) {
    *err = cat("head_dim ", dm.d, " unsupported (64, 128 or 256)");
    return P_UNSUPPORTED;
  }
  if (dm.hidden < 64 || dm.hidden % 64 != 0) {
    *err = cat("hidden ", dm.hidden, " must be a positive multiple of 64");
    return P_UNSUPPORTED;
  }
  if (dm.vocab < 2) {
    *err = cat("vocab ", dm.vocab, " must be >= 2");
    return P_INVALID;
  }
  if (dm.dtype != 0 && dm.dtype != 1) {
    *err = cat("dtype ", dm.dtype, " is neither SV_F32 (0) nor SV_BF16 (1)");
    return P_INVALID;
  }
  if (dm.max_rows < 1 || dm.max_roots < 1 || dm.max_pos < 1) {
    *err = "max_rows, max_roots and max_pos must be >= 1";
    return P_INVALID;
  }
  if (dm.max_tree_rows < 1 || dm.max_tree_rows > kMaxTreeRows) {
    *err = cat("max_tree_rows ", dm.max_tree_rows, " must be in [1, ", kMaxTreeRows, "]");
    return P_INVALID;
  }
  if (dm.weight_format != 0 && dm.weight_format != 1) {
    *err = cat("weight_format ", dm.weight_format, " is neither SV_WEIGHTS_NATIVE (0) nor SV_WEIGHTS_FP8 (1)");
    return P_INVALID;
  }
  if (dm.weight_format == 1 && dm.dtype != 1) {
    *err = "SV_WEIGHTS_FP8 takes bf16 models";
    return P_UNSUPPORTED;
  }
  if (dm.max_roots > dm.max_rows) {
    *err = "max_roots exceeds max_rows";
    return P_INVALID;
  }
  return P_OK;
}

const char *const kWideNames[RunPointers::kWide] = {"kv_k", "kv_v", "q_rows", "k_rows",
                                                    "v_rows", "drafter_logits", "logits"};
const char *const kNarrowNames[RunPointers::kNarrow] = {"draft_ids", "u_accept", "u_bonus", "accept_len",
                                                        "bonus",     "last_row", "surv_sum", "argmax",
                                                        "row_max",   "row_lse",  "overlap",  "survival"};

int check_alignment(const RunPointers &p, std::string *err) {
  for (int i = 0; i < RunPointers::kWide; ++i)
    if (reinterpret_cast<uintptr_t>(p.wide[i]) % 16 != 0) {
      *err = cat(kWideNames[i], " must be 16-byte aligned");
      return P_INVALID;
    }
  for (int i = 0; i < RunPointers::kNarrow; ++i)
    if (reinterpret_cast<uintptr_t>(p.narrow[i]) % 4 != 0) {
      *err = cat(kNarrowNames[i], " must be 4-byte aligned");
      return P_INVALID;
    }
  return P_OK;
}

// Up to 64 partial records per query vector, at least 16 Ki and at most
// 384 Ki records ((d + 2) floats each).
int64_t slot_capacity(const Dims &dm) {
  int64_t s = int64_t(64) * dm.Hq * dm.max_rows;
  return std::min<int64_t>(393216, std::max<int64_t>(16384, s));
}

static int qg_max_of(const Dims &dm) {
  const int G = dm.Hq / dm.Hkv;
  return int(ceil_div(int64_t(dm.max_tree_rows) * G, kItemQ));
}

MetaLayout meta_layout(int n, int R, int n_draft, int n_items, int n_runs, int n_groups) {
  MetaLayout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align16(o + bytes);
    return at;
  };
  L.row_tree = take(4 * size_t(n));
  L.row_local = take(4 * size_t(n));
  L.row_pos = take(4 * size_t(n));
  L.row_parent = take(4 * size_t(n));
  L.row_draft = take(4 * size_t(n));
  L.row_anc = take(8 * size_t(n));
  L.row_child = take(4 * size_t(n));
  L.draft_row = take(4 * size_t(std::max(n_draft, 1)));
  L.row_pack = take(4 * size_t(n));
  L.row_plocal = take(4 * size_t(n));
  L.row_klen = take(4 * size_t(n));
  L.row_panc = take(8 * size_t(n));
  L.tree_start = take(4 * size_t(R));
  L.tree_rows = take(4 * size_t(R));
  L.tree_kv_len = take(4 * size_t(R));
  L.tree_kv_off = take(8 * size_t(R));
  L.tree_done = take(4 * size_t(R));
  L.items = take(sizeof(AttnItem) * size_t(std::max(n_items, 1)));
  L.runs = take(sizeof(AttnRun) * size_t(std::max(n_runs, 1)));
  L.groups = take(sizeof(AttnGroup) * size_t(std::max(n_groups, 1)));
  L.total = o;
  return L;
}

size_t meta_capacity(const Dims &dm, int target_items) {
  const int qg = qg_max_of(dm);
  const int groups = dm.max_roots * dm.Hkv * qg;
  const int runs = std::max(target_items, 1);
  return meta_layout(dm.max_rows, dm.max_roots, dm.max_rows, runs + groups, runs, groups).total;
}

int build_plan(const Dims &dm, const HostInputs &in, int64_t slot_cap, int target_items,
               Plan *plan, std::string *err) {
  Plan &P = *plan;
  P = Plan{};
  if (in.n_rows < 1) {
    *err = cat("n_rows ", in.n_rows, " must be >= 1");
    return P_INVALID;
  }
  if (in.n_rows > dm.max_rows) {
    *err = cat("n_rows ", in.n_rows, " exceeds max_rows ", dm.max_rows);
    return P_CAPACITY;
  }
  if (in.n_roots < 1) {
    *err = cat("n_roots ", in.n_roots, " must be >= 1");
    return P_INVALID;
  }
  if (in.n_roots > dm.max_roots) {
    *err = cat("n_roots ", in.n_roots, " exceeds max_roots ", dm.max_roots);
    return P_CAPACITY;
  }
  if (!in.parent || !in.pos || !in.root_kv_off || !in.root_kv_len) {
    *err = "parent, pos, root_kv_off and root_kv_len must be non-null host arrays";
    return P_INVALID;
  }
  if (in.kv_tokens < 0) {
    *err = "kv_tokens must be >= 0";
    return P_INVALID;
  }
  const int n = in.n_rows;
  P.n = n;
  P.row_tree.resize(n);
  P.row_local.resize(n);
  P.row_pos.resize(n);
  P.row_parent.resize(n);
  P.row_draft.resize(n);
  P.row_anc.resize(n);
  int tree = -1, start = 0;
  for (int i = 0; i < n; ++i) {
    const int p = in.parent[i];
    if (p == -1) {
      ++tree;
      if (tree >= in.n_roots) {
        *err = cat("row ", i, " starts tree ", tree, " but n_roots is ", in.n_roots);
        return P_BAD_TREE;
      }
      start = i;
      P.tree_start.push_back(i);
    } else {
      if (i == 0) {
        *err = "row 0 must be a root (parent -1)";
        return P_BAD_TREE;
      }
      if (p < start || p >= i) {
        *err = cat("row ", i, ": parent ", p, " outside its tree's rows [", start, ", ", i, ")");
        return P_BAD_TREE;
      }
    }
    const int local = i - start;
    if (local >= dm.max_tree_rows) {
      *err = cat("tree ", tree, " has more than max_tree_rows = ", dm.max_tree_rows, " rows");
      return P_CAPACITY;
    }
    if (in.pos[i] < 0 || in.pos[i] >= dm.max_pos) {
      *err = cat("row ", i, ": position ", in.pos[i], " outside [0, max_pos = ", dm.max_pos, ")");
      return P_BAD_TREE;
    }
    P.row_tree[i] = tree;
    P.row_local[i] = local;
    P.row_pos[i] = in.pos[i];
    P.row_parent[i] = p;
    P.row_anc[i] = (p == -1 ? 0ull : P.row_anc[p]) | (1ull << local);
    if (p == -1) {
      P.row_draft[i] = -1;
    } else {
      P.row_draft[i] = int32_t(P.draft_row.size());
      P.draft_row.push_back(i);
    }
  }
  P.row_child.assign(n, -1);
  for (int i = 0; i < n; ++i) {
    const int p = P.row_parent[i];
    if (p >= 0) {
      if (P.row_child[p] >= 0) P.chains_only = false;
      P.row_child[p] = i;
    }
  }
  P.R = tree + 1;
  if (P.R != in.n_roots) {
    *err = cat("parent map has ", P.R, " roots but n_roots is ", in.n_roots);
    return P_BAD_TREE;
  }
  P.n_draft = int(P.draft_row.size());
  P.tree_rows.resize(P.R);
  P.tree_kv_len.resize(P.R);
  P.tree_kv_off.resize(P.R);
  for (int r = 0; r < P.R; ++r) {
    const int end = (r + 1 < P.R) ? P.tree_start[r + 1] : n;
    P.tree_rows[r] = end - P.tree_start[r];
    const int64_t off = in.root_kv_off[r];
    const int32_t len = in.root_kv_len[r];
    if (len < 0 || off < 0 || off + len > in.kv_tokens) {
      *err = cat("tree ", r, ": prefix [", off, ", ", off + int64_t(len), ") outside the ",
                 in.kv_tokens, " KV tokens");
      return P_BAD_TREE;
    }
    if (int64_t(len) + dm.max_pos > (int64_t(1) << 30)) {
      *err = cat("tree ", r, ": prefix length ", len, " too large");
      return P_CAPACITY;
    }
    P.tree_kv_len[r] = len;
    P.tree_kv_off[r] = off;
  }

  // ---- attention work list -------------------------------------------------
  const int G = dm.Hq / dm.Hkv;
  const int KT = attn_key_tile(dm.d);
  P.qg_max = qg_max_of(dm);
  // Packs: a tree joins the pack of the trees before it when it reads the
  // same KV segment (same offset), the pack stays within 64 rows (ancestor
  // bits) and kItemQ query vectors per KV head (one query group), and the
  // prefix lengths stay within a factor 2 (queries of the shorter trees run
  // over the longest prefix, masked).  Head dims above 128 keep one tree
  // per pack (their attention kernel has no register for a per-query prefix
  // length).
  std::vector<int32_t> pack_first, pack_start, pack_rows, pack_len, pack_min;
  std::vector<int64_t> pack_off;
  for (int r = 0; r < P.R;) {
    int rows = P.tree_rows[r], lo = P.tree_kv_len[r], hi = lo, e = r + 1;
    while (dm.d <= 128 && e < P.R && P.tree_kv_off[e] == P.tree_kv_off[r] && rows + P.tree_rows[e] <= 64 &&
           int64_t(rows + P.tree_rows[e]) * G <= kItemQ) {
      const int l2 = std::min(lo, P.tree_kv_len[e]), h2 = std::max(hi, P.tree_kv_len[e]);
      if (int64_t(h2) > 2 * int64_t(l2) + KT) break;
      rows += P.tree_rows[e];
      lo = l2;
      hi = h2;
      ++e;
    }
    pack_first.push_back(r);
    pack_start.push_back(P.tree_start[r]);
    pack_rows.push_back(rows);
    pack_len.push_back(hi);
    pack_min.push_back(lo);
    pack_off.push_back(P.tree_kv_off[r]);
    r = e;
  }
  const int NP = int(pack_first.size());
  P.n_packs = NP;
  P.row_pack.resize(n);
  P.row_plocal.resize(n);
  P.row_klen.resize(n);
  P.row_panc.resize(n);
  for (int pk = 0; pk < NP; ++pk)
    for (int i = pack_start[pk]; i < pack_start[pk] + pack_rows[pk]; ++i) {
      const int r = P.row_tree[i];
      P.row_pack[i] = pk;
      P.row_plocal[i] = i - pack_start[pk];
      P.row_klen[i] = P.tree_kv_len[r];
      P.row_panc[i] = P.row_anc[i] << (P.tree_start[r] - pack_start[pk]);
    }
  std::vector<int64_t> tiles(NP);
  int64_t total = 0;
  int mq_max = 1;
  for (int pk = 0; pk < NP; ++pk) {
    const int64_t len = pack_len[pk];
    // per-lane byte offsets into one pack's prefix stay below 2^31
    if (dm.dtype == 1 && (len + KT) * dm.Hkv * dm.d * 2 >= (int64_t(1) << 31)) {
      *err = cat("tree ", pack_first[pk], ": prefix length ", len, " too large for 32-bit KV offsets");
      return P_UNSUPPORTED;
    }
    tiles[pk] = ceil_div(len, KT) + ceil_div(pack_rows[pk], KT);
    const int64_t mq = int64_t(pack_rows[pk]) * G;
    mq_max = int(std::max<int64_t>(mq_max, std::min<int64_t>(mq, kItemQ)));
    total += int64_t(dm.Hkv) * ceil_div(mq, kItemQ) * tiles[pk];
  }
  // Runs: the sequence of every query group's tiles (group order: tree, KV
  // head, query group) cut into pieces of `chunk` tiles.  A run that covers a
  // group's tiles only in part shares that group with its neighbours; each
  // (run, group) pair is one work item.  Each item writes nq partial records
  // of (d + 2) floats: keep the run at least 4 * nq keys long, so that the
  // records stay below half of the K + V bytes a run reads, unless that
  // leaves fewer than target_items / 2 runs (one per compute unit: small,
  // latency-bound batches gain more from the parallelism than the records
  // cost); keep a group's items within kMaxSplits; aim for `target_items`
  // runs, and no more runs than workgroups the launch keeps resident
  // (target_items for four-wave workgroups, two per compute unit; half as
  // many for the eight-wave launch of groups with more than 64 query vectors,
  // one per compute unit), so that no compute unit takes a second round.
  int64_t max_tiles = 1;
  for (int pk = 0; pk < NP; ++pk) max_tiles = std::max(max_tiles, tiles[pk]);
  const int64_t per_cu = std::max(target_items / 2, 1);
  const int64_t resident = mq_max > 64 ? per_cu : std::max(target_items, 1);
  const int64_t rec_chunk = std::min(ceil_div(4 * int64_t(mq_max), KT), std::max<int64_t>(1, total / per_cu));
  int64_t chunk = std::max<int64_t>({ceil_div(64, KT), rec_chunk, ceil_div(total, resident),
                                     ceil_div(max_tiles, kMaxSplits - 1)});   // in tiles
  auto for_each_item = [&](int64_t ch, auto &&fn) {
    // fn(r, g, qg, m0, nq, tile0, tile1, run) for every work item in order
    int64_t at = 0;   // position in the whole sequence
    for (int r = 0; r < NP; ++r) {
      const int mq = pack_rows[r] * G;
      for (int g = 0; g < dm.Hkv; ++g)
        for (int qg = 0; qg * kItemQ < mq; ++qg) {
          const int m0 = qg * kItemQ;
          const int nq = std::min(kItemQ, mq - m0);
          for (int64_t t0 = 0; t0 < tiles[r];) {
            const int64_t run = at / ch;
            const int64_t t1 = std::min(tiles[r], t0 + (run + 1) * ch - at);
            fn(r, g, qg, m0, nq, t0, t1, run);
            at += t1 - t0;
            t0 = t1;
          }
        }
    }
  };
  for (;;) {
    int64_t slots = 0;
    for_each_item(chunk, [&](int, int, int, int, int nq, int64_t, int64_t, int64_t) { slots += nq; });
    if (slots <= slot_cap) break;
    if (chunk > (int64_t(1) << 30) / KT) {
      *err = "attention partial capacity exhausted";
      return P_CAPACITY;
    }
    chunk *= 2;
  }
  P.chunk = int32_t(chunk * KT);
  const int n_groups = P.R * dm.Hkv * P.qg_max;
  P.groups.assign(n_groups, AttnGroup{0, 0, 0, 0});
  P.runs.assign(size_t(ceil_div(total, chunk)), AttnRun{0, 0, 0, 0});
  int64_t slot = 0;
  for_each_item(chunk, [&](int r, int g, int qg, int m0, int nq, int64_t t0, int64_t t1, int64_t run) {
    const int gi = (r * dm.Hkv + g) * P.qg_max + qg;
    AttnGroup &Gr = P.groups[gi];
    if (Gr.count == 0) {
      Gr.first = int32_t(P.items.size());
      Gr.slot = int32_t(slot);
      Gr.nq = nq;
    }
    ++Gr.count;
    AttnRun &R = P.runs[size_t(run)];
    if (R.count == 0) R.first = int32_t(P.items.size());
    ++R.count;
    R.tiles += int32_t(t1 - t0);
    AttnItem it{};
    it.tree = r;
    it.g = g;
    it.m0 = m0;
    it.nq = nq;
    it.k0 = int32_t(t0 * KT);
    it.k1 = int32_t(t1 * KT);
    it.slot = int32_t(slot);
    it.tree_start = pack_start[r];
    it.tree_rows = pack_rows[r];
    it.kv_len = pack_len[r];
    it.kv_off = pack_off[r];
    it.kv_min = pack_min[r];
    slot += nq;
    P.items.push_back(it);
  });
  P.slots = slot;
  const size_t cap_runs = size_t(std::max(target_items, 1));
  if (P.runs.size() > cap_runs || P.items.size() > cap_runs + size_t(dm.max_roots) * dm.Hkv * P.qg_max ||
      P.slots > slot_cap) {
    *err = "attention work list exceeds the handle's capacity";
    return P_CAPACITY;
  }
  return P_OK;
}

void pack_plan(const Plan &p, int Hkv, void *dst, MetaLayout *lay) {
  const int n_groups = p.R * Hkv * p.qg_max;
  MetaLayout L = meta_layout(p.n, p.R, p.n_draft, int(p.items.size()), int(p.runs.size()), n_groups);
  char *b = static_cast<char *>(dst);
  auto put = [&](size_t off, const void *src, size_t bytes) {
    if (bytes) std::memcpy(b + off, src, bytes);
  };
  put(L.row_tree, p.row_tree.data(), 4 * size_t(p.n));
  put(L.row_local, p.row_local.data(), 4 * size_t(p.n));
  put(L.row_pos, p.row_pos.data(), 4 * size_t(p.n));
  put(L.row_parent, p.row_parent.data(), 4 * size_t(p.n));
  put(L.row_draft, p.row_draft.data(), 4 * size_t(p.n));
  put(L.row_anc, p.row_anc.data(), 8 * size_t(p.n));
  put(L.row_child, p.row_child.data(), 4 * size_t(p.n));
  put(L.draft_row, p.draft_row.data(), 4 * size_t(p.n_draft));
  put(L.row_pack, p.row_pack.data(), 4 * size_t(p.n));
  put(L.row_plocal, p.row_plocal.data(), 4 * size_t(p.n));
  put(L.row_klen, p.row_klen.data(), 4 * size_t(p.n));
  put(L.row_panc, p.row_panc.data(), 8 * size_t(p.n));
  put(L.tree_start, p.tree_start.data(), 4 * size_t(p.R));
  put(L.tree_rows, p.tree_rows.data(), 4 * size_t(p.R));
  put(L.tree_kv_len, p.tree_kv_len.data(), 4 * size_t(p.R));
  put(L.tree_kv_off, p.tree_kv_off.data(), 8 * size_t(p.R));
  std::memset(b + L.tree_done, 0, 4 * size_t(p.R));
  put(L.items, p.items.data(), sizeof(AttnItem) * p.items.size());
  put(L.runs, p.runs.data(), sizeof(AttnRun) * p.runs.size());
  put(L.groups, p.groups.data(), sizeof(AttnGroup) * size_t(n_groups));
  *lay = L;
}

}  // namespace sv
