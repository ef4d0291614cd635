// Test-only driver of the host planner and the verify-budget schedule, built
// with g++ -fsanitize=address,undefined by the CPU tests (no GPU, no HIP).
// Reads cases from the file named on the command line, one per line, and
// prints one result line per case:
//
//   P hq hkv d hidden vocab dtype max_rows max_roots max_tree_rows max_pos
//     n_rows n_roots kv_tokens slot_cap target  parent[n] pos[n] off[R] len[R]
//     -> "P <status> <items> <runs> <slots> <meta bytes> <sum of ancestor masks>"
//        (the plan is also serialised into a buffer of exactly its size)
//   A wide_misalign[7] narrow_misalign[12]   (byte offsets from an aligned base)
//     -> "A <status>"
//   S n_req n_cand[n_req] parent[K] conf[K] n_curve rows[n_curve] ms[n_curve]
//     max_rows  -> "S <status> <selected count> <expected tokens>"
#include <cstdio>
#include <cstdint>
#include <cstring>
#include <fstream>
#include <sstream>
#include <string>
#include <vector>

#include "plan.hpp"
#include "schedule.hpp"

namespace {

template <class T>
std::vector<T> take(std::istringstream &in, long n) {
  std::vector<T> v(size_t(n > 0 ? n : 0));
  for (auto &x : v) in >> x;
  return v;
}

}  // namespace

int main(int argc, char **argv) {
  if (argc < 2) return 2;
  std::ifstream f(argv[1]);
  std::string line;
  while (std::getline(f, line)) {
    if (line.empty()) continue;
    std::istringstream in(line);
    char kind = 0;
    in >> kind;
    if (kind == 'P') {
      sv::Dims dm{};
      in >> dm.Hq >> dm.Hkv >> dm.d >> dm.hidden >> dm.vocab >> dm.dtype >> dm.max_rows >> dm.max_roots >>
          dm.max_tree_rows >> dm.max_pos;
      int n = 0, R = 0, target = 0;
      long long kv = 0, slot_cap = 0;
      in >> n >> R >> kv >> slot_cap >> target;
      // exact-size heap copies, so that any read past an array is caught
      auto parent = take<int32_t>(in, n), pos = take<int32_t>(in, n);
      auto off = take<int64_t>(in, R);
      auto len = take<int32_t>(in, R);
      std::string err;
      int st = sv::check_dims(dm, &err);
      sv::Plan p;
      if (st == sv::P_OK) {
        sv::HostInputs hi{n, R, parent.data(), pos.data(), off.data(), len.data(), kv};
        st = sv::build_plan(dm, hi, slot_cap, target, &p, &err);
      }
      if (st != sv::P_OK) {
        std::printf("P %d\n", st);
        continue;
      }
      const sv::MetaLayout lay = sv::meta_layout(p.n, p.R, p.n_draft, int(p.items.size()), int(p.runs.size()),
                                                 p.R * dm.Hkv * p.qg_max);
      std::vector<char> buf(lay.total);
      sv::MetaLayout lay2{};
      sv::pack_plan(p, dm.Hkv, buf.data(), &lay2);
      unsigned long long anc = 0;
      for (uint64_t a : p.row_anc) anc += a;
      std::printf("P %d %zu %zu %lld %zu %llu\n", st, p.items.size(), p.runs.size(), (long long)p.slots, lay.total,
                  anc);
    } else if (kind == 'A') {
      alignas(16) static char base[64];
      sv::RunPointers rp{};
      for (int i = 0; i < sv::RunPointers::kWide; ++i) {
        int o = 0;
        in >> o;
        rp.wide[i] = base + o;
      }
      for (int i = 0; i < sv::RunPointers::kNarrow; ++i) {
        int o = 0;
        in >> o;
        rp.narrow[i] = base + o;
      }
      std::string err;
      std::printf("A %d\n", sv::check_alignment(rp, &err));
    } else if (kind == 'S') {
      int n_req = 0;
      in >> n_req;
      auto n_cand = take<int32_t>(in, n_req);
      long K = 0;
      for (int32_t c : n_cand) K += c > 0 ? c : 0;
      auto parent = take<int32_t>(in, K);
      auto conf = take<float>(in, K);
      int n_curve = 0;
      in >> n_curve;
      auto rows = take<int32_t>(in, n_curve);
      auto ms = take<float>(in, n_curve);
      int max_rows = 0;
      in >> max_rows;
      std::vector<int32_t> sel(size_t(K > 0 ? K : 1));
      double tok = 0, step = 0;
      std::string err;
      const int st = sv::schedule_budget(n_req, n_cand.data(), parent.data(), conf.data(), n_curve, rows.data(),
                                         ms.data(), max_rows, sel.data(), &tok, &step, &err);
      long cnt = 0;
      for (long k = 0; k < K; ++k) cnt += sel[size_t(k)];
      std::printf("S %d %ld %.9g\n", st, st == 0 ? cnt : 0L, st == 0 ? tok : 0.0);
    } else {
      return 3;
    }
  }
  return 0;
}
