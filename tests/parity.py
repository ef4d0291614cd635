"""Comparison of the HIP outputs with the oracle under the verify-step rules.

Tolerances (bf16 inputs, fp32 accumulation):
  * greedy token / bonus / accept length: exact where the oracle's top-2
    logit gap exceeds 1e-2 (for accept length: every row the walk consults);
    below that the GPU choice must be a near-maximal token of the oracle
    logits and the GPU walk must agree with the GPU's own greedy tokens;
  * logits: |d| <= 2e-2 * max(|ref|, rms(ref row));
  * probabilities p = softmax(logits): 1e-3 absolute;
  * overlaps and survival products: 2e-3 absolute.
"""
from __future__ import annotations

import numpy as np

GAP = 1e-2
LOGIT_REL = 2e-2
PROB_ABS = 1e-3
OV_ABS = 2e-3


def walk(parent, start, end, greedy, drafts):
    """Greedy walk over rows [start, end) with the given greedy tokens."""
    cur, acc = start, 0
    while True:
        nxt = None
        for c in range(cur + 1, end):
            if parent[c] == cur and drafts[c] == greedy[cur]:
                nxt = c
                break
        if nxt is None:
            return acc + 1, int(greedy[cur]), cur
        cur, acc = nxt, acc + 1


def tree_ranges(parent):
    roots = [i for i, p in enumerate(parent) if p < 0]
    return list(zip(roots, roots[1:] + [len(parent)]))


def check_self_consistency(parent, drafts, gpu, greedy=True):
    """Properties that hold at any size, from the GPU outputs alone (the
    greedy walk only when `greedy`)."""
    parent = np.asarray(parent)
    n = len(parent)
    ov, sv = gpu["overlap"], gpu["survival"]
    assert np.isfinite(ov).all() and np.isfinite(sv).all()
    assert (ov >= -1e-6).all() and (ov <= 1 + 2e-3).all(), (ov.min(), ov.max())
    assert (gpu["row_lse"] >= gpu["row_max"] - 1e-6).all()
    for t, (s, e) in enumerate(tree_ranges(list(parent))):
        assert ov[s] == 1.0 and sv[s] == 1.0
        surv = np.ones(e - s)
        for i in range(s + 1, e):
            surv[i - s] = surv[parent[i] - s] * np.float64(ov[i])
        np.testing.assert_allclose(sv[s:e], surv, rtol=1e-5, atol=1e-7)
        assert abs(gpu["surv_sum"][t] - surv[1:].sum()) <= 1e-5 * max(1.0, surv[1:].sum()) + 1e-6
        if greedy:
            acc, bonus, last = walk(parent, s, e, gpu["argmax"], drafts)
            assert (gpu["accept_len"][t], gpu["bonus"][t], gpu["last_row"][t]) == (acc, bonus, last), t
        depth = 0
        for i in range(s + 1, e):
            d, j = 0, i
            while parent[j] >= 0:
                j, d = parent[j], d + 1
            depth = max(depth, d)
        assert 1 <= gpu["accept_len"][t] <= depth + 1
    assert n == len(gpu["argmax"])


def compare(ref, gpu, parent, drafts, rows=None, logits_ref=None, logits_gpu=None, report=None, greedy=True):
    """Element-wise parity of the rows in `rows` (default all) and the trees
    that contain them (their greedy acceptance outputs when `greedy`).
    Returns a dict of the worst errors."""
    parent = list(np.asarray(parent))
    n = len(parent)
    rows = list(range(n)) if rows is None else list(rows)
    worst = {"argmax_mismatch_clear": 0, "near_ties": 0, "ov": 0.0, "surv": 0.0, "lse": 0.0,
             "logit": 0.0, "prob": 0.0}
    gap = ref["gap"]
    for i in rows:
        if gap[i] > GAP:
            if int(gpu["argmax"][i]) != int(ref["argmax"][i]):
                worst["argmax_mismatch_clear"] += 1
        else:
            worst["near_ties"] += 1
            if logits_ref is not None:
                # the GPU's choice must be one of the (near-)maximal tokens
                li = logits_ref[i]
                assert li[int(gpu["argmax"][i])] >= li.max() - GAP - 1e-9, i
        worst["ov"] = max(worst["ov"], abs(float(gpu["overlap"][i]) - ref["overlap"][i]))
        worst["surv"] = max(worst["surv"], abs(float(gpu["survival"][i]) - ref["survival"][i]))
        scale = max(1.0, abs(ref["row_lse"][i]))
        worst["lse"] = max(worst["lse"], abs(float(gpu["row_lse"][i]) - ref["row_lse"][i]) / scale,
                           abs(float(gpu["row_max"][i]) - ref["row_max"][i]) / scale)
    assert worst["argmax_mismatch_clear"] == 0, worst
    assert worst["ov"] <= OV_ABS, worst
    assert worst["surv"] <= OV_ABS, worst
    assert worst["lse"] <= LOGIT_REL, worst
    if logits_ref is not None and logits_gpu is not None:
        for i in rows:
            lr, lg = logits_ref[i], logits_gpu[i].astype(np.float64)
            rms = np.sqrt(np.mean(lr * lr))
            err = np.abs(lg - lr) / np.maximum(np.abs(lr), rms)
            worst["logit"] = max(worst["logit"], float(err.max()))
            pr = np.exp(lr - ref["row_lse"][i])
            pg = np.exp(lg - float(gpu["row_lse"][i]))
            worst["prob"] = max(worst["prob"], float(np.abs(pr - pg).max()))
        assert worst["logit"] <= LOGIT_REL, worst
        assert worst["prob"] <= PROB_ABS, worst
    # trees fully inside `rows`: acceptance outputs
    rs = set(rows)
    for t, (s, e) in enumerate(tree_ranges(parent)):
        if not all(i in rs for i in range(s, e)):
            continue
        assert abs(float(gpu["surv_sum"][t]) - ref["surv_sum"][t]) <= OV_ABS * (e - s), (t, gpu["surv_sum"][t], ref["surv_sum"][t])
        if not greedy:
            continue
        # rows the oracle's walk consults: accepted rows (their argmax decides)
        acc, bonus, last = int(ref["accept_len"][t]), int(ref["bonus"][t]), int(ref["last_row"][t])
        path = []
        j = last
        while j >= 0:
            path.append(j)
            j = parent[j]
        if all(gap[j] > GAP for j in path):
            assert (int(gpu["accept_len"][t]), int(gpu["bonus"][t]), int(gpu["last_row"][t])) == (acc, bonus, last), t
        else:
            worst["near_ties"] += 1
    if report is not None:
        report.update(worst)
    return worst


def _softmax64(x):
    x = np.asarray(x, np.float64)
    e = np.exp(x - x.max())
    return e / e.sum()


def check_sample(parent, drafts, u_accept, u_bonus, logits_ref, drafter_ref, gpu, trees=None, report=None):
    """T = 1 acceptance outputs of the GPU against the oracle's fp64
    distributions.  Along the GPU's walk, each accept test u * q(d) < p(d)
    must go the oracle's way unless the two sides are within the logit
    tolerance of each other in log terms (|ln(u q) - ln p| <= 2 LOGIT_REL
    max(|l_d|, rms of the row's logits): the test then may go either way);
    the walk must stop where the oracle rejects (or at a leaf), and the bonus
    token t must satisfy C(t-1) - tol <= u_bonus <= C(t) + tol for the
    oracle's normalised running weights C of the GPU's stop row, with tol =
    OV_ABS (a CDF value is a sum of probabilities, like the overlap).
    `drafter_ref[k]` are the drafter logits of the k-th draft row.  Returns
    the number of trees whose walk had no near decision and matched
    `ref`-style exact outputs."""
    parent = list(np.asarray(parent))
    n = len(parent)
    child = [-1] * n
    for i, p in enumerate(parent):
        if p >= 0:
            assert child[p] < 0, "chains only"
            child[p] = i
    draft_index = {}
    for i, p in enumerate(parent):
        if p >= 0:
            draft_index[i] = len(draft_index)
    worst = {"near_decisions": 0, "draw_slack": 0.0, "walks": 0}
    for t, (s, e) in enumerate(tree_ranges(parent)):
        if trees is not None and t not in trees:
            continue
        acc, last, bonus = int(gpu["accept_len"][t]), int(gpu["last_row"][t]), int(gpu["bonus"][t])
        cur, k = s, 0

        def decision(cur, c):
            lc = np.asarray(logits_ref[cur], np.float64)
            d = int(drafts[c])
            p = _softmax64(lc)[d]
            q = _softmax64(drafter_ref[draft_index[c]])[d]
            lhs, rhs = float(u_accept[c]) * q, p
            rms = float(np.sqrt(np.mean(lc * lc)))
            delta = 2 * LOGIT_REL * max(abs(float(lc[d])), rms)
            if lhs == 0.0:
                return True, True
            near = abs(np.log(lhs) - np.log(rhs)) <= delta
            return lhs < rhs, not near

        while k < acc - 1:
            c = child[cur]
            assert c >= 0, (t, "GPU walk past a leaf")
            ok, clear = decision(cur, c)
            if clear:
                assert ok, (t, cur, c, "GPU accepted where the oracle rejects")
            else:
                worst["near_decisions"] += 1
            cur, k = c, k + 1
        assert last == cur, (t, last, cur)
        c = child[cur]
        if c >= 0:
            ok, clear = decision(cur, c)
            if clear:
                assert not ok, (t, cur, c, "GPU rejected where the oracle accepts")
            else:
                worst["near_decisions"] += 1
        p = _softmax64(logits_ref[cur])
        w = np.maximum(p - _softmax64(drafter_ref[draft_index[c]]), 0.0) if c >= 0 else p
        if w.sum() <= 0:
            w = p
        cdf = np.cumsum(w) / w.sum()
        lo = float(cdf[bonus - 1]) if bonus > 0 else 0.0
        hi = float(cdf[bonus])
        u = float(u_bonus[t])
        slack = max(lo - u, u - hi, 0.0)
        worst["draw_slack"] = max(worst["draw_slack"], slack)
        assert slack <= OV_ABS, (t, bonus, lo, u, hi)
        worst["walks"] += 1
    if report is not None:
        report.update(worst)
    return worst
