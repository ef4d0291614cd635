"""Plain, slow fp64 CPU oracle for one verify step of a parallel draft block.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this module.  It shares no code with
the HIP library (no kernels, headers, helpers or tables); it reads the same
seeded inputs and nothing else.

What it computes, step by step (every float in fp64, inputs decoded exactly
from their fp32 / bf16 bits):

1. Tree layout.  Rows form a forest of contiguous trees, each starting at its
   root (parent -1); a node's parent lies earlier in the same tree.  A row's
   visible rows are its ancestors and itself (SpecOPD summary, onedev.kr,
   section "what differs": ancestor-and-self tree mask fed by a parent map).
2. Rotary positions.  Row queries and row keys are rotated by their semantic
   position, not by their packed index (same section).  NeoX half-split pairs
   (k, k+d/2) with angle pos * base^(-2k/d).  Prefix keys are a cache written
   in earlier steps, already rotated.
3. Attention.  Query head h uses KV head floor(h / (Hq/Hkv)); scores
   q.k / sqrt(d) over prefix[off:off+len] plus the ancestor-or-self rows; a
   max-subtracted softmax; output = weighted sum of values.
4. Projection h = W_o . concat(o), then a unit-gain RMS norm
   h / sqrt(mean(h^2) + eps) (the target has a final norm before its head:
   sionic.ai Solar Open2 page, section 3, hidden taken before the final norm).
5. LM head logits = W_lm . h over the full vocabulary (Dev.to/aiwithghost
   DSpine page, file-contents section: the head spans the whole vocabulary).
   p = softmax(logits); greedy token = lowest index of the maximum.
6. Overlap of draft row i (parent j) = sum_u min(p_j(u), q_i(u)) with
   q_i = softmax(drafter logits of i); equal to 1 - TV(p_j, q_i)
   (SpecOPD summary, "how it is used"; VESSL part 2, DSpark section:
   alpha = 1 - D_TV).  Roots: 1.
7. Acceptance per tree (sionic.ai page, section 1; VESSL part 2, Blockwise
   section: verify in one forward, keep the longest matching prefix): walk
   from the root, repeatedly step to the first child (row order) whose draft
   id equals the current row's greedy token.  accept_len counts the accepted
   drafts plus the bonus token (SpecOPD summary, "premises and limits"), the
   bonus is the greedy token of the last accepted row.
8. Prefix survival: survival(root) = 1, survival(i) = survival(parent) *
   overlap(i) (SpecOPD summary, "how it is used": product of the acceptance
   probabilities of the earlier positions); surv_sum = sum over non-root rows
   of the tree (the expected accepted length a scheduler obtains by
   multiplying probabilities, VESSL part 2, DSpark section).
9. T = 1 stochastic verification of chains (mode 1).  The pages evaluate
   sampling at T = 1 (DSpine page, temperature section; SpecOPD summary,
   "premises and limits") and give the per-position acceptance probability
   as alpha = 1 - D_TV (VESSL part 2, DSpark section) without writing the
   rule out; the plainest rule with exactly that acceptance is the standard
   one taken here: at row cur with child c carrying draft d, accept when
   u_accept[c] * q_c(d) < p_cur(d) (probability min(1, p/q)); on the first
   rejection the bonus token is drawn from max(0, p_cur - q_c), and when the
   walk reaches a leaf it is drawn from p_cur, both by the inverse CDF at
   u_bonus (the smallest token whose running weight exceeds u_bonus times
   the total; a residual without mass falls back to p_cur).  The uniforms
   are inputs.  Trees with branching nodes are not taken in this mode.  A
   draft id outside the vocabulary is a token neither model can emit
   (p = q = 0 there), so the test 0 < 0 fails and it is rejected, as it is
   in greedy mode, where it never equals a greedy token.
10. Commit (the step after verify: sionic.ai page, section 1, generation
   resumes after the matching leading drafts; section 6, committing accepted
   tokens follows verify).  Each tree's accepted path, its root and then
   every accepted draft in depth order (accept_len rows, ending at last_row),
   joins the tree's cache right after its visible prefix: entry off + len + j
   holds the j-th path row's key rotated at its semantic position and its
   value, in the cache's number format (bf16 or fp32).  The bonus token is
   not committed; it is the root of the next step, at the position after the
   last committed row, seeing len + accept_len cache entries.
11. FP8 LM head (weight format "fp8"; the pages' fastest serving runs the
   target in FP8: sionic.ai page, section 5).  W8A8 in OCP e4m3 (4 exponent
   bits, bias 7, 3 mantissa bits, largest finite 448, subnormal step 2^-9,
   no infinities), values rounded to nearest, ties to even.  Each LM-head
   row n gets the power-of-two scale s_n = 2^e, e the smallest integer with
   max_k |W[n, k]| <= 448 * 2^e (1 for a zero row), and at least -126, so
   that every scale is a normal fp32 number; each normalised hidden row t
   likewise a_t from max |h_t|.  q = e4m3(value / scale) (an exact
   division), and logits[t, n] = a_t s_n sum_k q_h[t, k] q_w[n, k].
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------------------
# input decoding (the oracle's own)
# ----------------------------------------------------------------------------


def decode(x, dtype: str) -> np.ndarray:
    """Exact fp64 value of a tensor given as bf16 bit patterns or as fp32."""
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


# ----------------------------------------------------------------------------
# 1. tree layout
# ----------------------------------------------------------------------------


class Forest:
    """Rows partitioned into contiguous trees (parent map + row order)."""

    def __init__(self, parent):
        parent = [int(p) for p in parent]
        n = len(parent)
        self.parent = parent
        self.n = n
        self.roots = []          # root row of each tree, in order
        self.tree_of = [0] * n
        self.draft_index = [-1] * n
        nd = 0
        for i, p in enumerate(parent):
            if p == -1:
                self.roots.append(i)
            else:
                if not self.roots:
                    raise ValueError("first row must be a root")
                start = self.roots[-1]
                if not (start <= p < i):
                    raise ValueError(f"row {i}: parent {p} outside [{start},{i})")
                self.draft_index[i] = nd
                nd += 1
            self.tree_of[i] = len(self.roots) - 1
        if n and not self.roots:
            raise ValueError("no root")
        self.n_draft = nd
        ends = self.roots[1:] + [n]
        self.tree_rows = [list(range(s, e)) for s, e in zip(self.roots, ends)]

    def path(self, i: int) -> list:
        """Rows from the tree's root down to i, inclusive (ancestors-or-self)."""
        out = [i]
        while self.parent[out[-1]] != -1:
            out.append(self.parent[out[-1]])
        return out[::-1]

    def children(self, i: int) -> list:
        t = self.tree_of[i]
        return [c for c in self.tree_rows[t] if self.parent[c] == i]


# ----------------------------------------------------------------------------
# 2. rotary positions
# ----------------------------------------------------------------------------


def rope(x: np.ndarray, pos, base: float) -> np.ndarray:
    """Rotate the last axis of x (length d) by position `pos`.

    Pair k couples components k and k + d/2 and turns by angle
    pos * base^(-2k/d), k = 0 .. d/2-1."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    k = np.arange(half, dtype=np.float64)
    theta = np.power(float(base), -2.0 * k / d)
    ang = float(pos) * theta
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


# ----------------------------------------------------------------------------
# 3. attention
# ----------------------------------------------------------------------------


def attend(q: np.ndarray, keys: np.ndarray, values: np.ndarray) -> np.ndarray:
    """q [Hq, d]; keys, values [L, Hkv, d] (L >= 1).  Returns o [Hq, d]."""
    Hq, d = q.shape
    Hkv = keys.shape[1]
    group = Hq // Hkv
    o = np.empty((Hq, d))
    for h in range(Hq):
        g = h // group
        s = keys[:, g, :] @ q[h] / np.sqrt(d)
        w = np.exp(s - s.max())
        w = w / w.sum()
        o[h] = w @ values[:, g, :]
    return o


# ----------------------------------------------------------------------------
# 5. softmax statistics
# ----------------------------------------------------------------------------


def row_stats(logits: np.ndarray):
    """max, logsumexp, greedy token (lowest index of the max) and the gap
    between the largest and second-largest logit of one row."""
    m = float(logits.max())
    lse = m + float(np.log(np.exp(logits - m).sum()))
    arg = int(np.argmax(logits))          # first occurrence = lowest index
    if logits.shape[0] > 1:
        top2 = np.partition(logits, -2)[-2:]
        gap = float(top2[1] - top2[0])
    else:
        gap = float("inf")
    return m, lse, arg, gap


def softmax(logits: np.ndarray) -> np.ndarray:
    m = logits.max()
    e = np.exp(logits - m)
    return e / e.sum()


# ----------------------------------------------------------------------------
# 6.-8. overlap, acceptance, survival
# ----------------------------------------------------------------------------


def overlap(p: np.ndarray, q: np.ndarray) -> float:
    """sum_u min(p(u), q(u))."""
    return float(np.minimum(p, q).sum())


def accept_walk(forest: Forest, root: int, greedy, draft_ids):
    """Greedy longest-matching walk from `root`.  Returns
    (accept_len, bonus, last_row); accept_len includes the bonus token."""
    cur, acc = root, 0
    while True:
        nxt = None
        for c in forest.children(cur):
            if int(draft_ids[c]) == int(greedy[cur]):
                nxt = c
                break
        if nxt is None:
            break
        cur, acc = nxt, acc + 1
    return acc + 1, int(greedy[cur]), cur


def survival(forest: Forest, overlaps):
    """survival(root) = 1; survival(i) = survival(parent(i)) * overlap(i).
    Returns (survival per row, surv_sum per tree)."""
    s = np.zeros(forest.n)
    for i in range(forest.n):
        p = forest.parent[i]
        s[i] = 1.0 if p == -1 else s[p] * overlaps[i]
    sums = np.array([sum(s[i] for i in rows if forest.parent[i] != -1)
                     for rows in forest.tree_rows])
    return s, sums


# ----------------------------------------------------------------------------
# 9. T = 1 stochastic verification (chains)
# ----------------------------------------------------------------------------


def sample_inverse_cdf(weights: np.ndarray, u: float):
    """Smallest token t whose running weight sum exceeds u * (total weight),
    for non-negative weights with a positive total and u in [0, 1).  Also
    returns the distance from u * total to the nearest running sum (relative
    to the total), which says how close the draw is to a neighbouring token."""
    c = np.cumsum(np.asarray(weights, dtype=np.float64))
    z = float(c[-1])
    target = u * z
    t = int(np.searchsorted(c, target, side="right"))
    lo = float(c[t - 1]) if t > 0 else 0.0
    margin = min(target - lo, float(c[t]) - target) / z
    return t, margin


def stochastic_walk(forest: Forest, root: int, p_of, q_of, draft_ids, u_accept, u_bonus: float):
    """T = 1 walk of one chain from `root` (step 9).  p_of(row) is the
    target distribution at a row, q_of(row) the drafter distribution of a
    non-root row.  Returns (accept_len, bonus, last_row, margin) where margin
    is the smallest relative distance of any accept test, or of the bonus
    draw, from its decision boundary."""
    cur, acc = root, 0
    margin = float("inf")
    while True:
        ch = forest.children(cur)
        if len(ch) > 1:
            raise ValueError(f"row {cur} has {len(ch)} children: stochastic verification takes chains")
        p = p_of(cur)
        if not ch:
            t, m = sample_inverse_cdf(p, u_bonus)
            return acc + 1, t, cur, min(margin, m)
        c = ch[0]
        d = int(draft_ids[c])
        q = q_of(c)
        inside = 0 <= d < len(p)
        lhs = float(u_accept[c]) * float(q[d]) if inside else 0.0
        rhs = float(p[d]) if inside else 0.0
        margin = min(margin, abs(lhs - rhs) / max(rhs, lhs, 1e-300))
        if lhs < rhs:
            cur, acc = c, acc + 1
            continue
        resid = np.maximum(p - q, 0.0)
        t, m = sample_inverse_cdf(resid if resid.sum() > 0 else p, u_bonus)
        return acc + 1, t, cur, min(margin, m)


# ----------------------------------------------------------------------------
# the whole step
# ----------------------------------------------------------------------------


def attention_outputs(cfg, inp, rows) -> dict:
    """Steps 2-3 for the listed rows.

    `cfg` needs n_q_heads, n_kv_heads, head_dim, rope_base, dtype; `inp`
    needs parent, pos, root_kv_off, root_kv_len, kv_k, kv_v, q_rows, k_rows,
    v_rows.  Returns {row: o (fp64 [Hq, d])}.
    """
    dt = cfg["dtype"]
    forest = Forest(inp["parent"])
    pos = [int(p) for p in inp["pos"]]
    base = cfg["rope_base"]
    out = {}
    by_tree = {}
    for i in rows:
        by_tree.setdefault(forest.tree_of[i], []).append(i)
    for t, trows in by_tree.items():
        # the tree's prefix, decoded once for all of its rows
        off = int(inp["root_kv_off"][t])
        ln = int(inp["root_kv_len"][t])
        pre_k = decode(inp["kv_k"][off:off + ln], dt)
        pre_v = decode(inp["kv_v"][off:off + ln], dt)
        for i in trows:
            anc = forest.path(i)
            row_k = np.stack([rope(decode(inp["k_rows"][a], dt), pos[a], base) for a in anc])
            row_v = np.stack([decode(inp["v_rows"][a], dt) for a in anc])
            keys = np.concatenate([pre_k, row_k], axis=0)
            vals = np.concatenate([pre_v, row_v], axis=0)
            q = rope(decode(inp["q_rows"][i], dt), pos[i], base)
            out[i] = attend(q, keys, vals)
    return out


def project_norm(w_o: np.ndarray, o: np.ndarray, eps: float) -> np.ndarray:
    """Step 4: h = W_o . concat_h(o_h), then h / sqrt(mean(h^2) + eps)."""
    h = w_o @ o.reshape(-1)
    return h / np.sqrt(np.mean(h * h) + eps)


def hidden_states(cfg, inp, rows) -> dict:
    """Steps 2-4: {row: normalised hidden state (fp64 [hidden])}."""
    w_o = decode(inp["w_o"], cfg["dtype"])
    att = attention_outputs(cfg, inp, rows)
    return {i: project_norm(w_o, att[i], cfg["norm_eps"]) for i in rows}


def e4m3(x) -> np.ndarray:
    """Nearest OCP e4m3 value (ties to even) of each |x| <= 448, as fp64."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(a > 448.0):
        raise ValueError("e4m3 takes |x| <= 448")
    _, ex = np.frexp(np.where(a > 0, a, 1.0))        # a = m 2^ex, m in [0.5, 1)
    step = np.where(a < 2.0 ** -6, 2.0 ** -9, np.ldexp(1.0, ex - 4))   # 3 mantissa bits below 2^(ex-1)
    return np.sign(x) * np.round(a / step) * step     # np.round: half to even


def pow2_scale(amax: float) -> float:
    """Smallest 2^e, e >= -126, with amax <= 448 * 2^e (1 when amax is 0)."""
    if amax == 0.0:
        return 1.0
    e = int(np.ceil(np.log2(amax / 448.0)))
    while amax > 448.0 * 2.0 ** e:
        e += 1
    while amax <= 448.0 * 2.0 ** (e - 1):
        e -= 1
    return 2.0 ** max(e, -126)


def pow2_scales(amax) -> np.ndarray:
    """pow2_scale of each entry (vectorised: the same smallest power of two)."""
    amax = np.asarray(amax, dtype=np.float64)
    pos = amax > 0
    e = np.ceil(np.log2(np.where(pos, amax, 448.0) / 448.0))
    e = np.where(amax > 448.0 * np.exp2(e), e + 1, e)
    e = np.where(amax <= 448.0 * np.exp2(e - 1), e - 1, e)
    return np.where(pos, np.exp2(np.maximum(e, -126.0)), 1.0)


def lm_head_fp8(cfg, w_lm, hs: np.ndarray, chunk: int = 8192, scales=None) -> np.ndarray:
    """Step 11: logits [m, V] of the W8A8 e4m3 LM head.  `scales` forces the
    hidden rows' scales (the other valid outcome when a row's largest value
    sits on a scale boundary)."""
    a = pow2_scales(np.abs(hs).max(axis=1)) if len(hs) else np.zeros(0)
    if scales is not None:
        # a forced scale may be the next lower power of two, where the row's
        # largest values sit just past 448: they are held at +-448
        a = np.asarray(scales, dtype=np.float64)
        qh = e4m3(np.clip(hs / a[:, None], -448.0, 448.0))
    else:
        qh = e4m3(hs / a[:, None]) if len(hs) else hs
    V = w_lm.shape[0]
    out = np.empty((hs.shape[0], V))
    for lo in range(0, V, chunk):
        w = decode(w_lm[lo:lo + chunk], cfg["dtype"])
        sw = pow2_scales(np.abs(w).max(axis=1))
        qw = e4m3(w / sw[:, None])
        out[:, lo:lo + chunk] = (qh @ qw.T) * a[:, None] * sw[None, :]
    return out


def lm_head(cfg, w_lm, hs: np.ndarray, chunk: int = 8192) -> np.ndarray:
    """logits [m, V] = hs [m, hidden] . W_lm^T, decoding W_lm chunk by chunk."""
    V = w_lm.shape[0]
    out = np.empty((hs.shape[0], V))
    for lo in range(0, V, chunk):
        w = decode(w_lm[lo:lo + chunk], cfg["dtype"])
        out[:, lo:lo + chunk] = hs @ w.T
    return out


def verify(cfg, inp, trees=None, keep_logits: bool = False) -> dict:
    """Run the whole verify step for the listed trees (default: all).

    Rows outside the listed trees get NaN / -1 in the outputs.
    Returns a dict of numpy arrays: argmax, row_max, row_lse, gap, overlap,
    survival per row; accept_len, bonus, last_row, surv_sum per tree (with
    inp["mode"] == 1, the T = 1 walk of step 9 on inp["u_accept"] and
    inp["u_bonus"], and walk_margin, its closest decision); optionally
    logits [n, V] (NaN for rows not computed)."""
    forest = Forest(inp["parent"])
    n, R = forest.n, len(forest.roots)
    if trees is None:
        trees = list(range(R))
    rows = [i for t in trees for i in forest.tree_rows[t]]
    hs = hidden_states(cfg, inp, rows)
    H = np.stack([hs[i] for i in rows]) if rows else np.zeros((0, 1))
    head = lm_head_fp8 if cfg.get("weight_format") == "fp8" else lm_head
    logits = head(cfg, inp["w_lm"], H) if rows else np.zeros((0, 0))
    V = logits.shape[1] if rows else 0

    res = {k: np.full(n, np.nan) for k in ("row_max", "row_lse", "gap", "overlap", "survival")}
    res["argmax"] = np.full(n, -1, np.int64)
    for r_idx, i in enumerate(rows):
        m, lse, arg, gap = row_stats(logits[r_idx])
        res["row_max"][i], res["row_lse"][i] = m, lse
        res["argmax"][i], res["gap"][i] = arg, gap

    where = {i: r_idx for r_idx, i in enumerate(rows)}
    dl = inp["drafter_logits"]
    for i in rows:
        j = forest.parent[i]
        if j == -1:
            res["overlap"][i] = 1.0
            continue
        p = softmax(logits[where[j]])
        q = softmax(decode(dl[forest.draft_index[i]], cfg["dtype"]))
        res["overlap"][i] = overlap(p, q)

    surv_all, _ = survival(forest, np.where(np.isnan(res["overlap"]), 0.0, res["overlap"]))
    for k in ("accept_len", "bonus", "last_row"):
        res[k] = np.full(R, -1, np.int64)
    res["surv_sum"] = np.full(R, np.nan)
    res["walk_margin"] = np.full(R, np.inf)
    for t in trees:
        for i in forest.tree_rows[t]:
            res["survival"][i] = surv_all[i]
        if int(inp.get("mode", 0)) == 1:
            def p_of(i):
                return softmax(logits[where[i]])

            def q_of(i):
                return softmax(decode(dl[forest.draft_index[i]], cfg["dtype"]))

            acc, bonus, last, mg = stochastic_walk(forest, forest.roots[t], p_of, q_of, inp["draft_ids"],
                                                   inp["u_accept"], float(inp["u_bonus"][t]))
            res["walk_margin"][t] = mg
        else:
            acc, bonus, last = accept_walk(forest, forest.roots[t], res["argmax"], inp["draft_ids"])
        res["accept_len"][t], res["bonus"][t], res["last_row"][t] = acc, bonus, last
        res["surv_sum"][t] = sum(surv_all[i] for i in forest.tree_rows[t] if forest.parent[i] != -1)
    if keep_logits:
        full = np.full((n, V), np.nan)
        for r_idx, i in enumerate(rows):
            full[i] = logits[r_idx]
        res["logits"] = full
    res["rows"] = np.array(rows, np.int64)
    return res


def target_greedy(cfg, inp, trees=None) -> np.ndarray:
    """Greedy token per row (the target's argmax), -1 where not computed."""
    return verify(cfg, inp, trees)["argmax"]


def cfg_dict(cfg) -> dict:
    """The scalar model description the oracle needs, from any object with the
    usual attribute names."""
    return {"dtype": cfg.dtype, "n_q_heads": cfg.n_q_heads, "n_kv_heads": cfg.n_kv_heads,
            "head_dim": cfg.head_dim, "rope_base": cfg.rope_base, "norm_eps": cfg.norm_eps}


def inp_dict(inp) -> dict:
    """The tensors the oracle reads, from a generated input set."""
    st = inp.st
    return {"parent": st.parent, "pos": st.pos, "root_kv_off": st.root_kv_off,
            "root_kv_len": st.root_kv_len, "kv_k": inp.kv_k, "kv_v": inp.kv_v,
            "q_rows": inp.q_rows, "k_rows": inp.k_rows, "v_rows": inp.v_rows,
            "w_o": inp.w_o, "w_lm": inp.w_lm, "drafter_logits": inp.drafter_logits,
            "draft_ids": inp.draft_ids}


# ----------------------------------------------------------------------------
# 10. commit and the next step's layout
# ----------------------------------------------------------------------------


def to_cache_format(x, dtype: str) -> np.ndarray:
    """fp64 values as stored in the cache: fp32 by round-to-nearest-even; for
    bf16, that fp32 rounded to nearest-even on its upper 16 bits, returned as
    the bf16 bit patterns (uint16)."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype != "bf16":
        return f
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def commit(cfg, inp, res, kv_k, kv_v):
    """Step 10 for every tree: returns copies of (kv_k, kv_v) with the
    accepted paths written after the visible prefixes.  `res` gives
    accept_len and last_row per tree; `inp` the step's structure and rows."""
    dt = cfg["dtype"]
    forest = Forest(inp["parent"])
    kk = np.array(kv_k, copy=True)
    vv = np.array(kv_v, copy=True)
    for t in range(len(forest.roots)):
        acc, last = int(res["accept_len"][t]), int(res["last_row"][t])
        path = forest.path(last)
        if len(path) != acc:
            raise ValueError(f"tree {t}: last_row {last} is at depth {len(path) - 1}, accept_len {acc}")
        end = int(inp["root_kv_off"][t]) + int(inp["root_kv_len"][t])
        for j, row in enumerate(path):
            k = rope(decode(inp["k_rows"][row], dt), int(inp["pos"][row]), cfg["rope_base"])
            kk[end + j] = to_cache_format(k, dt)
            vv[end + j] = inp["v_rows"][row]
    return kk, vv


def advance(inp, res, gamma: int):
    """Layout of the next chain step after a commit: tree t keeps its cache
    offset, sees len + accept_len entries, and its new root (the bonus token)
    sits at the position after the last committed row, followed by gamma
    draft rows.  Returns (parent, pos, root_kv_off, root_kv_len)."""
    forest = Forest(inp["parent"])
    parent, pos, lens = [], [], []
    for t, root in enumerate(forest.roots):
        acc = int(res["accept_len"][t])
        p0 = int(inp["pos"][root]) + acc
        start = len(parent)
        for i in range(gamma + 1):
            parent.append(-1 if i == 0 else start + i - 1)
            pos.append(p0 + i)
        lens.append(int(inp["root_kv_len"][t]) + acc)
    return (np.array(parent, np.int32), np.array(pos, np.int32),
            np.array(inp["root_kv_off"], np.int64), np.array(lens, np.int32))
