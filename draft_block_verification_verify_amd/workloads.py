"""Seeded synthetic inputs for one verify step of a parallel draft block.

This module only draws random numbers and lays out tree structure.  It holds
none of the verify step's arithmetic (no attention, no projection, no softmax,
no acceptance rule); both the HIP path and the CPU oracle take their inputs
from here.

Workloads (all shapes from the five verify configurations this library is
measured on):

  chain-tiny      fp32, 1 chain, prefix 128, gamma 7, 4/2 heads, d 64,
                  hidden 256, vocab 4096 ("Tiny chain verify").
  chain-8b        bf16, 1 chain, prefix 4096, gamma 7, 32/8 heads, d 128,
                  hidden 4096, vocab 151,936 (Qwen3-8B-shaped full attention).
  block-27b-b16   bf16, 1 chain, prefix 8192, 16 drafts, 24/4 heads, d 256,
                  hidden 5120, vocab 248,320 (27B shape, b16 block as on the
                  DSpine-b16 card, Dev.to/aiwithghost page, TL;DR).
  tree-specopd    bf16, shared stem 2048, 64 anchors x 7-token branches,
                  32/8 heads, d 128, hidden 4096, vocab 151,936 (proposal tree
                  of the SpecOPD summary, onedev.kr page, "how it works").
  conc32-27b      bf16, 32 chains with ragged prefixes U{1024..16384},
                  gamma 7, 27B shape.

Distributions: activations and KV ~ N(0,1); W_o ~ N(0, 1/sqrt(Hq*d));
LM head ~ N(0, 0.02) (N(0, 1/16) for the fp32 chain); drafter logits
~ N(0, 2) (the second argument of N(.,.) is a standard deviation).
bf16 tensors are fp32 normals rounded to nearest-even and are passed around
as their uint16 bit patterns, so both sides see identical bits.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field

import numpy as np

# ----------------------------------------------------------------------------
# configurations
# ----------------------------------------------------------------------------


@dataclass(frozen=True)
class Config:
    cfg_id: int
    name: str
    dtype: str            # "f32" or "bf16"
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    hidden: int
    vocab: int
    kind: str             # "chain", "tree", "multichain"
    prefix: int = 0       # chain: prefix length
    gamma: int = 7        # drafts per chain / per branch
    n_seqs: int = 1       # multichain: number of sequences
    min_len: int = 0      # multichain: ragged prefix range (inclusive)
    max_len: int = 0
    stem: int = 0         # tree: shared stem length
    anchors: int = 0      # tree: number of anchors B
    branch_w: int = 0     # tree: tokens per branch W (root + W-1 drafts)
    w_lm_std: float = 0.02
    rope_base: float = 10000.0
    norm_eps: float = 1e-6

    @property
    def w_o_std(self) -> float:
        return 1.0 / np.sqrt(self.n_q_heads * self.head_dim)


CONFIGS: dict[int, Config] = {
    1: Config(1, "chain-tiny", "f32", 4, 2, 64, 256, 4096, "chain",
              prefix=128, gamma=7, w_lm_std=1.0 / 16.0),
    2: Config(2, "chain-8b", "bf16", 32, 8, 128, 4096, 151936, "chain",
              prefix=4096, gamma=7),
    3: Config(3, "block-27b-b16", "bf16", 24, 4, 256, 5120, 248320, "chain",
              prefix=8192, gamma=16),
    4: Config(4, "tree-specopd", "bf16", 32, 8, 128, 4096, 151936, "tree",
              stem=2048, anchors=64, branch_w=7, gamma=6),
    5: Config(5, "conc32-27b", "bf16", 24, 4, 256, 5120, 248320, "multichain",
              gamma=7, n_seqs=32, min_len=1024, max_len=16384),
}

# tensor tags for independent random streams
_TAG = {"kv_k": 1, "kv_v": 2, "q": 3, "k": 4, "v": 5, "w_o": 6, "w_lm": 7,
        "drafter": 8, "struct": 9, "plant": 10, "sample": 11, "uniform": 12}


def _rng(cfg_id: int, seed: int, tag: str, sub: int = 0, rnd: int = 0) -> np.random.Generator:
    key = [cfg_id, seed, _TAG[tag], sub] + ([rnd] if rnd else [])
    return np.random.default_rng(key)


# ----------------------------------------------------------------------------
# number formats
# ----------------------------------------------------------------------------


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest-even) and return the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


_POOL_WORKERS = max(1, min(16, os.cpu_count() or 1))


def _normal(cfg: Config, seed: int, tag: str, shape, std: float, rnd: int = 0) -> np.ndarray:
    """N(0, std^2) of `shape` in the config dtype (uint16 bits for bf16).

    Large tensors are drawn in fixed 4M-element chunks, each from its own
    stream, so the values do not depend on the thread count.  `rnd` > 0
    selects the streams of step `rnd` of a multi-step run.
    """
    total = int(np.prod(shape))
    chunk = 1 << 22
    nchunks = max(1, (total + chunk - 1) // chunk)
    out = np.empty(total, dtype=np.uint16 if cfg.dtype == "bf16" else np.float32)

    def fill(c: int) -> None:
        lo = c * chunk
        hi = min(total, lo + chunk)
        r = _rng(cfg.cfg_id, seed, tag, c, rnd)
        v = r.standard_normal(hi - lo, dtype=np.float32) * np.float32(std)
        out[lo:hi] = f32_to_bf16_bits(v) if cfg.dtype == "bf16" else v

    if nchunks == 1:
        fill(0)
    else:
        with _cf.ThreadPoolExecutor(_POOL_WORKERS) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


# ----------------------------------------------------------------------------
# structure
# ----------------------------------------------------------------------------


@dataclass
class Structure:
    parent: np.ndarray        # int32 [n]  (-1 = root)
    pos: np.ndarray           # int32 [n]  semantic position
    root_kv_off: np.ndarray   # int64 [R]
    root_kv_len: np.ndarray   # int32 [R]
    kv_tokens: int
    anchors: np.ndarray | None = None   # tree workloads only

    @property
    def n_rows(self) -> int:
        return int(self.parent.shape[0])

    @property
    def n_roots(self) -> int:
        return int(self.root_kv_off.shape[0])


def chain_structure(prefix_lens, gamma, slack: int = 0) -> Structure:
    """Independent chains: sequence s = root (last committed token) + gamma
    drafts (`gamma` an int, or one count per sequence).

    Each sequence owns a KV segment of L_s + slack entries (the slack takes
    committed rows of later steps); its rows sit at positions L_s, L_s+1,
    ..., L_s+gamma_s.
    """
    parent, pos, offs, lens = [], [], [], []
    off = 0
    gammas = [int(gamma)] * len(prefix_lens) if np.isscalar(gamma) else [int(g) for g in gamma]
    for L, g in zip(prefix_lens, gammas):
        start = len(parent)
        for i in range(g + 1):
            parent.append(-1 if i == 0 else start + i - 1)
            pos.append(int(L) + i)
        offs.append(off)
        lens.append(int(L))
        off += int(L) + int(slack)
    return Structure(np.array(parent, np.int32), np.array(pos, np.int32),
                     np.array(offs, np.int64), np.array(lens, np.int32), off)


def tree_structure(stem: int, anchors, branch_w: int) -> Structure:
    """Proposal tree: one shared stem; branch b = anchor row at a_b seeing
    stem[0:a_b], then branch_w-1 drafted rows at a_b+1 .. a_b+branch_w-1."""
    parent, pos, offs, lens = [], [], [], []
    for a in anchors:
        start = len(parent)
        for j in range(branch_w):
            parent.append(-1 if j == 0 else start + j - 1)
            pos.append(int(a) + j)
        offs.append(0)
        lens.append(int(a))
    return Structure(np.array(parent, np.int32), np.array(pos, np.int32),
                     np.array(offs, np.int64), np.array(lens, np.int32), stem,
                     anchors=np.asarray(anchors, np.int64))


def make_structure(cfg: Config, seed: int, slack: int = 0) -> Structure:
    r = _rng(cfg.cfg_id, seed, "struct")
    if cfg.kind == "chain":
        return chain_structure([cfg.prefix], cfg.gamma, slack)
    if cfg.kind == "multichain":
        lens = r.integers(cfg.min_len, cfg.max_len + 1, size=cfg.n_seqs)
        return chain_structure(lens, cfg.gamma, slack)
    if slack:
        raise ValueError("slack applies to chain workloads")
    if cfg.kind == "tree":
        a = np.sort(r.choice(np.arange(1, cfg.stem + 1), size=cfg.anchors,
                             replace=False))
        return tree_structure(cfg.stem, a, cfg.branch_w)
    raise ValueError(cfg.kind)


def draft_rows(parent: np.ndarray) -> np.ndarray:
    """Indices of the non-root rows, in row order (the drafter-logit rows)."""
    return np.nonzero(np.asarray(parent) >= 0)[0]


# ----------------------------------------------------------------------------
# full input set
# ----------------------------------------------------------------------------


@dataclass
class Inputs:
    cfg: Config
    seed: int
    st: Structure
    kv_k: np.ndarray          # [kv_tokens, Hkv, d]
    kv_v: np.ndarray
    q_rows: np.ndarray        # [n, Hq, d]
    k_rows: np.ndarray        # [n, Hkv, d]
    v_rows: np.ndarray
    w_o: np.ndarray           # [hidden, Hq*d]
    w_lm: np.ndarray          # [V, hidden]
    drafter_logits: np.ndarray  # [n_draft, V]
    draft_ids: np.ndarray     # int32 [n]; root entries 0
    extras: dict = field(default_factory=dict)


def make_inputs(cfg_id: int | Config, seed: int = 0, *, with_weights: bool = True, slack: int = 0) -> Inputs:
    cfg = cfg_id if isinstance(cfg_id, Config) else CONFIGS[cfg_id]
    st = make_structure(cfg, seed, slack)
    n, Hq, Hkv, d = st.n_rows, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    n_draft = int((st.parent >= 0).sum())
    T = max(st.kv_tokens, 0)
    kv_k = _normal(cfg, seed, "kv_k", (T, Hkv, d), 1.0)
    kv_v = _normal(cfg, seed, "kv_v", (T, Hkv, d), 1.0)
    q = _normal(cfg, seed, "q", (n, Hq, d), 1.0)
    k = _normal(cfg, seed, "k", (n, Hkv, d), 1.0)
    v = _normal(cfg, seed, "v", (n, Hkv, d), 1.0)
    if with_weights:
        w_o = _normal(cfg, seed, "w_o", (cfg.hidden, Hq * d), cfg.w_o_std)
        w_lm = _normal(cfg, seed, "w_lm", (cfg.vocab, cfg.hidden), cfg.w_lm_std)
    else:
        w_o = w_lm = None
    dl = _normal(cfg, seed, "drafter", (n_draft, cfg.vocab), 2.0)
    draft_ids = np.zeros(n, np.int32)
    return Inputs(cfg, seed, st, kv_k, kv_v, q, k, v, w_o, w_lm, dl, draft_ids)


def round_rows(cfg: Config, seed: int, rnd: int, n_rows: int, n_draft: int) -> dict:
    """Row tensors of step `rnd` >= 1 of a multi-step run (step 0 uses those
    of make_inputs): fresh q, k, v rows and drafter logits, same
    distributions, streams of their own."""
    Hq, Hkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    return {"q_rows": _normal(cfg, seed, "q", (n_rows, Hq, d), 1.0, rnd),
            "k_rows": _normal(cfg, seed, "k", (n_rows, Hkv, d), 1.0, rnd),
            "v_rows": _normal(cfg, seed, "v", (n_rows, Hkv, d), 1.0, rnd),
            "drafter_logits": _normal(cfg, seed, "drafter", (n_draft, cfg.vocab), 2.0, rnd)}


def make_weights(cfg_id: int | Config, seed: int = 0):
    cfg = cfg_id if isinstance(cfg_id, Config) else CONFIGS[cfg_id]
    w_o = _normal(cfg, seed, "w_o", (cfg.hidden, cfg.n_q_heads * cfg.head_dim), cfg.w_o_std)
    w_lm = _normal(cfg, seed, "w_lm", (cfg.vocab, cfg.hidden), cfg.w_lm_std)
    return w_o, w_lm


# ----------------------------------------------------------------------------
# draft ids
# ----------------------------------------------------------------------------


def plant_chain_drafts(inp: Inputs, target_argmax: np.ndarray, *,
                       k_per_tree=None, rnd: int = 0) -> np.ndarray:
    """Plant chain drafts: per sequence draw k ~ U{0..gamma}; drafts 1..k copy
    the target's greedy token at the parent row, draft k+1 (if any) is uniform
    over the vocabulary minus that token, later drafts are uniform.

    `target_argmax` is whatever the caller uses as the target's greedy token
    per row.  `rnd` > 0 draws the plants of step `rnd` of a multi-step run.
    Returns k per tree and writes inp.draft_ids in place.
    """
    st, V = inp.st, inp.cfg.vocab
    r = _rng(inp.cfg.cfg_id, inp.seed, "plant", 0, rnd)
    roots = np.nonzero(st.parent < 0)[0]
    ends = list(roots[1:]) + [st.n_rows]
    ids = np.zeros(st.n_rows, np.int32)
    ks = []
    for t, (s, e) in enumerate(zip(roots, ends)):
        depth = e - s - 1
        k = int(r.integers(0, depth + 1)) if k_per_tree is None else int(k_per_tree[t])
        ks.append(k)
        for j in range(1, depth + 1):
            i = s + j
            par = st.parent[i]
            greedy = int(target_argmax[par])
            if j <= k:
                ids[i] = greedy
            elif j == k + 1:
                x = int(r.integers(0, V - 1))
                ids[i] = x if x < greedy else x + 1
            else:
                ids[i] = int(r.integers(0, V))
    inp.draft_ids = ids
    return np.array(ks, np.int32)


def sample_tree_drafts(inp: Inputs) -> np.ndarray:
    """Draft ids drawn from the drafter's own distribution softmax(b_i) with
    the Gumbel-max construction: id = argmax_u (b_iu + G_u), G ~ Gumbel(0,1)."""
    st, V = inp.st, inp.cfg.vocab
    rows = draft_rows(st.parent)
    ids = np.zeros(st.n_rows, np.int32)
    for t, i in enumerate(rows):
        r = _rng(inp.cfg.cfg_id, inp.seed, "sample", t)
        g = -np.log(-np.log(r.random(V)))
        b = (bf16_bits_to_f32(inp.drafter_logits[t]) if inp.cfg.dtype == "bf16"
             else inp.drafter_logits[t]).astype(np.float64)
        ids[i] = int(np.argmax(b + g))
    inp.draft_ids = ids
    return ids


def make_uniforms(inp: Inputs):
    """Uniforms in [0, 1) for the T = 1 verification rule: one accept test
    per non-root row (u_accept[n], roots 0) and one bonus draw per tree
    (u_bonus[R]), fp32 so that both sides read the same values."""
    st = inp.st
    r = _rng(inp.cfg.cfg_id, inp.seed, "uniform")
    u_accept = r.random(st.n_rows, dtype=np.float32)
    u_accept[np.asarray(st.parent) < 0] = 0.0
    u_bonus = r.random(st.n_roots, dtype=np.float32)
    return u_accept, u_bonus
