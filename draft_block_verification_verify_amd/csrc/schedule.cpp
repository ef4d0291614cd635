// Verify budget over a batch (VESSL AI "Speculative Decoding Part 2", DSpark
// section: per-position pass probabilities, multiplied into expected
// lengths, decide how much of the batch's verify budget each request gets,
// against a measured hardware curve; EAGLE-2 on the same page: a branch's
// score is the product of confidences along its path).
//
// A candidate's score is the probability that it is accepted; it never
// exceeds its parent's (conf <= 1).  For a budget of m draft rows the best
// selection is the m highest scores (ties: lower request, then lower index),
// which contains every member's parent; the step then yields n_req + (their
// sum) tokens in curve(n_req + m) ms, and the schedule takes the m with the
// most tokens per ms (the smallest such m on ties).
#include "schedule.hpp"

#include <algorithm>
#include <cmath>
#include <numeric>
#include <sstream>
#include <vector>

#include "plan.hpp"

namespace sv {

namespace {
template <class... A>
std::string cat(A &&...a) {
  std::ostringstream s;
  (s << ... << a);
  return s.str();
}
}  // namespace

double curve_step_ms(int n_curve, const int32_t *x, const float *y, double rows) {
  if (rows <= x[0] || n_curve == 1) return double(y[0]);
  for (int i = 1; i < n_curve; ++i) {
    if (rows <= x[i]) {
      const double t = (rows - x[i - 1]) / double(x[i] - x[i - 1]);
      return double(y[i - 1]) + t * (double(y[i]) - double(y[i - 1]));
    }
  }
  const int l = n_curve - 1;
  return double(y[l]) + (rows - x[l]) * (double(y[l]) - double(y[l - 1])) / double(x[l] - x[l - 1]);
}

int schedule_budget(int n_req, const int32_t *n_cand, const int32_t *cand_parent, const float *cand_conf,
                    int n_curve, const int32_t *curve_rows, const float *curve_ms, int max_rows,
                    int32_t *selected, double *expected_tokens, double *step_ms, std::string *err) {
  if (n_req < 1 || !n_cand) {
    *err = "n_req must be >= 1 and n_cand non-null";
    return P_INVALID;
  }
  if (n_curve < 1 || !curve_rows || !curve_ms) {
    *err = "the hardware curve needs at least one point";
    return P_INVALID;
  }
  for (int i = 0; i < n_curve; ++i) {
    if (curve_rows[i] < 1 || (i && curve_rows[i] <= curve_rows[i - 1])) {
      *err = "curve_rows must be >= 1 and strictly increasing";
      return P_INVALID;
    }
    if (!(curve_ms[i] > 0.0f) || !std::isfinite(curve_ms[i]) || (i && curve_ms[i] < curve_ms[i - 1])) {
      *err = "curve_ms must be positive, finite and non-decreasing";
      return P_INVALID;
    }
  }
  if (max_rows > 0 && max_rows < n_req) {
    *err = cat("max_rows ", max_rows, " is below the ", n_req, " root rows");
    return P_CAPACITY;
  }
  // scores (candidates of request r at offsets [off[r], off[r] + n_cand[r]))
  int64_t total = 0;
  for (int r = 0; r < n_req; ++r) {
    if (n_cand[r] < 0) {
      *err = cat("request ", r, ": n_cand < 0");
      return P_INVALID;
    }
    total += n_cand[r];
  }
  if (total > 0 && (!cand_parent || !cand_conf || !selected)) {
    *err = "cand_parent, cand_conf and selected must be non-null";
    return P_INVALID;
  }
  std::vector<double> score(static_cast<size_t>(total), 0.0);
  int64_t off = 0;
  for (int r = 0; r < n_req; ++r) {
    for (int k = 0; k < n_cand[r]; ++k) {
      const int p = cand_parent[off + k];
      const float c = cand_conf[off + k];
      if (!(p == -1 || (p >= 0 && p < k))) {
        *err = cat("request ", r, " candidate ", k, ": parent ", p, " is neither -1 nor an earlier candidate");
        return P_BAD_TREE;
      }
      if (!(c >= 0.0f && c <= 1.0f)) {
        *err = cat("request ", r, " candidate ", k, ": confidence ", c, " outside [0, 1]");
        return P_INVALID;
      }
      score[off + k] = double(c) * (p < 0 ? 1.0 : score[off + p]);
    }
    off += n_cand[r];
  }
  std::vector<int64_t> order(static_cast<size_t>(total));
  std::iota(order.begin(), order.end(), int64_t(0));
  std::stable_sort(order.begin(), order.end(), [&](int64_t a, int64_t b) { return score[a] > score[b]; });
  int64_t m_max = total;
  if (max_rows > 0) m_max = std::min<int64_t>(m_max, int64_t(max_rows) - n_req);
  double best_v = -1.0, best_tok = 0.0, best_ms = 0.0, sum = 0.0;
  int64_t best_m = 0;
  for (int64_t m = 0; m <= m_max; ++m) {
    if (m) sum += score[order[m - 1]];
    const double tok = double(n_req) + sum;
    const double ms = curve_step_ms(n_curve, curve_rows, curve_ms, double(n_req + m));
    const double v = tok / ms;
    if (v > best_v) {
      best_v = v;
      best_tok = tok;
      best_ms = ms;
      best_m = m;
    }
  }
  for (int64_t i = 0; i < total; ++i) selected[i] = 0;
  for (int64_t i = 0; i < best_m; ++i) selected[order[i]] = 1;
  if (expected_tokens) *expected_tokens = best_tok;
  if (step_ms) *step_ms = best_ms;
  return P_OK;
}

}  // namespace sv
