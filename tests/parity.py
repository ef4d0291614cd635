"""Comparison of the HIP outputs with the oracle under the verify-step rules.

Tolerances (bf16 inputs, fp32 accumulation):
  * greedy token / bonus / accept length: exact where the oracle's top-2
    logit gap exceeds 1e-2 (for accept length: every row the walk consults);
    below that the GPU choice must be a near-maximal token of the oracle
    logits and the GPU walk must agree with the GPU's own greedy tokens;
  * logits: |d| <= 2e-2 * max(|ref|, rms(ref row));
  * probabilities p = softmax(logits): 1e-3 absolute.  Without a logits
    buffer this is checked on the top token from the row statistics alone:
    p_max = exp(row_max - row_lse) moves by p_max * |d(row_max - row_lse)|,
    held to 1e-3; row_lse itself is held to 1e-3 absolute (an lse error d
    moves every p = exp(l - lse) by about p * d <= d, so this bounds what
    lse alone can do to any probability by the probability tolerance);
  * overlaps and survival products: 2e-3 absolute.

FP8 LM head (e4m3 W8A8): the activations are quantised from each side's own
hidden state, which differ by up to ~1e-3 relative (the bf16 pipeline
upstream, about uniform in size over a row).  An element whose scaled
value lies within EPS_H (2e-3) times the row's rms of an e4m3 rounding
midpoint may take the neighbouring code on the GPU, one e4m3 step away.  Per logit n of row t the two results may then
differ by B[t, n] = a_t * sum over such elements k of step_k * |s_n q_w[n, k]|
(fp8_bounds, from the oracle's own hidden state and weights); the logits are
held to B plus 1e-3 * max(|ref|, rms) (fp32 accumulation), decisions are
exact where the oracle's top-2 gap exceeds 2 max_n B[t, n] + 1e-2.  Since
lse moves by at most max_n B[t, n], the log-sum-exp is held to 1e-3 + max B
and each probability p_n to 1e-3 + p_n (exp(B[t, n] + max B) - 1) (the
top token's likewise, from the row statistics).  A row whose largest value sits within 1e-2 of a
scale boundary (448 * 2^e) may take the other power of two: it is held to
the nearer of the two references (fp8_alternatives).  Overlaps and survival
keep 2e-3.
"""
from __future__ import annotations

import numpy as np

GAP = 1e-2
LOGIT_REL = 2e-2
PROB_ABS = 1e-3
OV_ABS = 2e-3
EPS_H = 2e-3
LSE_ABS = 1e-3
FP8_TOL = {}


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


def fp8_bounds(cfg, inp, rows, eps=EPS_H, chunk=8192):
    """{row: B} with B[n] the largest |GPU - oracle| FP8 logit difference that
    activation code flips can make (see the module docstring)."""
    from oracle import verify_oracle as O
    hs = O.hidden_states(cfg, inp, rows)
    amb = []
    for i in rows:
        h = hs[i]
        a = O.pow2_scale(float(np.abs(h).max()))
        x = np.abs(h / a)
        _, ex = np.frexp(np.where(x > 0, x, 1.0))
        step = np.where(x < 2.0 ** -6, 2.0 ** -9, np.ldexp(1.0, ex - 4))
        mid = (np.floor(x / step) + 0.5) * step          # the rounding midpoint in x's step
        near = np.abs(x - mid) <= eps * np.sqrt(np.mean(x * x))   # the upstream error is about uniform in size
        amb.append(np.where(near, step * a, 0.0))
    amb = np.stack(amb)                                    # [rows, K]
    w_lm = inp["w_lm"]
    B = np.zeros((len(rows), w_lm.shape[0]))
    for lo in range(0, w_lm.shape[0], chunk):
        w = O.decode(w_lm[lo:lo + chunk], cfg["dtype"])
        sw = O.pow2_scales(np.abs(w).max(axis=1))
        wdq = np.abs(O.e4m3(w / sw[:, None]) * sw[:, None])
        B[:, lo:lo + chunk] = amb @ wdq.T
    return {i: B[r] for r, i in enumerate(rows)}


def _near_scale_boundary(h, rel):
    from oracle import verify_oracle as O
    amax = float(np.abs(h).max())
    s = O.pow2_scale(amax)
    return amax >= 448.0 * s * (1 - rel) or amax <= 448.0 * s / 2 * (1 + rel)


def plant_fp8_margins(cfg, inp, rows, margin=1.5, seed=0, rel=1e-2):
    """Give each listed row a clear FP8 decision.

    First, a row whose hidden state has its largest |value| within `rel` of a
    scale boundary (see fp8_alternatives) gets a fresh query vector (a row's
    query enters only its own attention output), up to 8 draws.  Then row i
    gets a token u_i (distinct per row) whose LM-head row moves along column
    i of the pseudo-inverse of the rows' hidden states H (the oracle's, fp64),
    so that logit u_i of row i rises to the row's largest logit + `margin`
    and the other listed rows' logits of u_i keep their values (H G = I;
    needs no more rows than the hidden width).  Writes inp.q_rows and
    inp.w_lm (bf16 bits) in place and returns the tokens.  The margin is in
    logit units, several times the FP8 flip bound (about 0.2 of the logits'
    rms)."""
    from oracle import verify_oracle as O
    from draft_block_verification_verify_amd import workloads as W
    cd = {"dtype": cfg["dtype"], "n_q_heads": cfg["n_q_heads"], "n_kv_heads": cfg["n_kv_heads"],
          "head_dim": cfg["head_dim"], "rope_base": cfg["rope_base"], "norm_eps": cfg["norm_eps"]}
    rows = list(rows)
    hs = O.hidden_states(cd, O.inp_dict(inp), rows)
    rq = np.random.default_rng([seed, 778])
    for _ in range(8):
        redo = [i for i in rows if _near_scale_boundary(hs[i], rel)]
        if not redo:
            break
        for i in redo:
            q = rq.standard_normal(inp.q_rows[i].shape).astype(np.float32)
            inp.q_rows[i] = W.f32_to_bf16_bits(q) if cd["dtype"] == "bf16" else q
        hs.update(O.hidden_states(cd, O.inp_dict(inp), redo))
    H = np.stack([hs[i] for i in rows])
    assert H.shape[0] <= H.shape[1], "more rows than the hidden width"
    lg = O.lm_head(cd, inp.w_lm, H)
    G = np.linalg.pinv(H)
    toks = np.random.default_rng([seed, 777]).choice(inp.w_lm.shape[0], size=len(rows), replace=False)
    w = O.decode(inp.w_lm[toks], cd["dtype"])
    delta = lg.max(axis=1) + margin - lg[np.arange(len(rows)), toks]
    w_new = w + (G * delta[None, :]).T
    inp.w_lm[toks] = W.f32_to_bf16_bits(w_new.astype(np.float32))
    return toks


def fp8_clear_fraction(ref, rows, bound, alt, gap=GAP):
    """Fraction of the listed rows whose FP8 decision is held exactly by
    compare(): oracle top-2 gap above 2 max B + gap and no second valid
    scale."""
    clear = [i for i in rows if i not in alt and ref["gap"][i] > gap + 2 * float(bound[i].max())]
    return len(clear) / max(1, len(rows))


def fp8_alternatives(cfg, inp, rows, rel=1e-2):
    """Rows whose oracle hidden state has its largest |value| within `rel`
    of a scale boundary (448 * 2^e): the GPU's own hidden state may take the
    neighbouring power of two, a different but valid quantisation.  Returns
    {row: oracle FP8 logits of the row at that other scale}."""
    from oracle import verify_oracle as O
    hs = O.hidden_states(cfg, inp, rows)
    alt_rows, alt_scale = [], []
    for i in rows:
        amax = float(np.abs(hs[i]).max())
        s = O.pow2_scale(amax)
        if amax >= 448.0 * s * (1 - rel):
            alt_rows.append(i)
            alt_scale.append(2 * s)
        elif amax <= 448.0 * s / 2 * (1 + rel):
            alt_rows.append(i)
            alt_scale.append(s / 2)
    if not alt_rows:
        return {}
    lg = O.lm_head_fp8(cfg, inp["w_lm"], np.stack([hs[i] for i in alt_rows]), scales=alt_scale)
    return {i: lg[k] for k, i in enumerate(alt_rows)}


def compare(ref, gpu, parent, drafts, rows=None, logits_ref=None, logits_gpu=None, report=None, greedy=True,
            tol=None, alt=None, bound=None):
    """Element-wise parity of the rows in `rows` (default all) and the trees
    that contain them (their greedy acceptance outputs when `greedy`).
    Returns a dict of the worst errors.  `tol` overrides gap / logit_rel /
    prob_abs (FP8_TOL for the FP8 LM head).  `alt` ({row: logits}) gives a
    second valid reference for some rows (fp8_alternatives): their values are
    held to the nearer reference and their decisions are treated like near
    ties (the GPU's choice must be near-maximal in one of the two).  `bound`
    ({row: B}) replaces the relative logit tolerance of those rows by B +
    1e-3 * max(|ref|, rms) and widens their decision gap to 2 max B + gap."""
    tol = tol or {}
    alt = alt or {}
    bound = bound or {}
    worst_alt = 0
    gap_t, logit_t, prob_t = tol.get("gap", GAP), tol.get("logit_rel", LOGIT_REL), tol.get("prob_abs", PROB_ABS)
    parent = list(np.asarray(parent))
    n = len(parent)
    rows = list(range(n)) if rows is None else list(rows)
    lse_t = tol.get("lse_abs", LSE_ABS)
    worst = {"argmax_mismatch_clear": 0, "near_ties": 0, "ov": 0.0, "surv": 0.0, "lse": 0.0,
             "top_prob": 0.0, "logit": 0.0, "prob": 0.0}
    gap = ref["gap"]

    def lse_max(x):
        m = float(np.max(x))
        return m + float(np.log(np.sum(np.exp(x - m)))), m

    def gap_of(i):
        return gap_t + (2 * float(bound[i].max()) if i in bound else 0.0)

    for i in rows:
        if i in alt:
            worst_alt += 1
            worst["near_ties"] += 1
            if logits_ref is not None:
                a = int(gpu["argmax"][i])
                assert any(li[a] >= li.max() - gap_t - 1e-9 for li in (logits_ref[i], alt[i])), i
        elif gap[i] > gap_of(i):
            if int(gpu["argmax"][i]) != int(ref["argmax"][i]):
                worst["argmax_mismatch_clear"] += 1
        else:
            worst["near_ties"] += 1
            if logits_ref is not None:
                # the GPU's choice must be one of the (near-)maximal tokens
                li = logits_ref[i]
                assert li[int(gpu["argmax"][i])] >= li.max() - gap_of(i) - 1e-9, i
        worst["ov"] = max(worst["ov"], abs(float(gpu["overlap"][i]) - ref["overlap"][i]))
        worst["surv"] = max(worst["surv"], abs(float(gpu["survival"][i]) - ref["survival"][i]))
        refs = [(ref["row_lse"][i], ref["row_max"][i])] + ([lse_max(alt[i])] if i in alt else [])
        gl, gm = float(gpu["row_lse"][i]), float(gpu["row_max"][i])
        bmax = float(bound[i].max()) if i in bound else 0.0
        # (with a flip bound: the excess over what code flips can move)
        e_lse = min(abs(gl - l) for l, m in refs) - bmax
        # the top token's probability from the row statistics alone
        e_top = min(abs(np.exp(gm - gl) - np.exp(m - l)) - np.exp(m - l) * np.expm1(2 * bmax) for l, m in refs)
        worst["lse"] = max(worst["lse"], e_lse)
        worst["top_prob"] = max(worst["top_prob"], e_top)
    assert worst["argmax_mismatch_clear"] == 0, worst
    assert worst["ov"] <= OV_ABS, worst
    assert worst["surv"] <= OV_ABS, worst
    assert worst["lse"] <= lse_t, worst
    assert worst["top_prob"] <= prob_t, worst
    if logits_ref is not None and logits_gpu is not None:
        for i in rows:
            lg = logits_gpu[i].astype(np.float64)
            pg = np.exp(lg - float(gpu["row_lse"][i]))
            e_logit, e_prob = np.inf, np.inf
            for lr in [logits_ref[i]] + ([alt[i]] if i in alt else []):
                rms = np.sqrt(np.mean(lr * lr))
                pr = np.exp(lr - lse_max(lr)[0])
                if i in bound:   # excess over the flip bound
                    err = np.maximum(np.abs(lg - lr) - bound[i], 0.0) / np.maximum(np.abs(lr), rms)
                    perr = np.abs(pr - pg) - pr * np.expm1(bound[i] + float(bound[i].max()))
                else:
                    err = np.abs(lg - lr) / np.maximum(np.abs(lr), rms)
                    perr = np.abs(pr - pg)
                if float(err.max()) < e_logit:
                    e_logit, e_prob = float(err.max()), float(perr.max())
            key = "logit_over_bound" if i in bound else "logit"
            worst[key] = max(worst.get(key, 0.0), e_logit)
            worst["prob"] = max(worst["prob"], e_prob)
        assert worst["logit"] <= logit_t, worst
        assert worst.get("logit_over_bound", 0.0) <= 1e-3, worst
        assert worst["prob"] <= prob_t, worst
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
        if all(gap[j] > gap_of(j) and j not in alt for j in path):
            assert (int(gpu["accept_len"][t]), int(gpu["bonus"][t]), int(gpu["last_row"][t])) == (acc, bonus, last), t
        else:
            worst["near_ties"] += 1
    worst["scale_boundary_rows"] = worst_alt
    if report is not None:
        report.update(worst)
    return worst


def sampled_trees(st, k=8):
    """k trees of a full-size batch for the oracle to score: the first, middle
    and last, the longest and the shortest prefix, and seeded others."""
    R = st.n_roots
    lens = np.asarray(st.root_kv_len)
    want = {0, R // 2, R - 1, int(np.argmax(lens)), int(np.argmin(lens))}
    r = np.random.default_rng(R)
    while len(want) < min(k, R):
        want.add(int(r.integers(0, R)))
    return sorted(want)


def walk_decisions(ref, gpu, parent, gap=GAP):
    """Per tree (accept_len, bonus, last_row): the oracle's where every row
    its walk consults has a top-2 gap above `gap` (compare() has asserted the
    GPU equal there), the GPU's at a near tie (where either choice is
    valid).  Returns the dict and the number of trees taken from the GPU."""
    parent = list(np.asarray(parent))
    out = {k: np.array(ref[k], copy=True) for k in ("accept_len", "bonus", "last_row")}
    from_gpu = 0
    for t, (s, e) in enumerate(tree_ranges(parent)):
        j, clear = int(ref["last_row"][t]), True
        while j >= 0:
            clear = clear and ref["gap"][j] > gap
            j = parent[j]
        if not clear:
            from_gpu += 1
            for k in out:
                out[k][t] = gpu[k][t]
    return out, from_gpu


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
            if not 0 <= d < len(lc):
                return False, True            # a token outside the vocabulary: rejected
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
