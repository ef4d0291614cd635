"""Algorithmic byte and flop counts of one verify step (for roofline figures).

"Algorithmic" means what the method must move or compute at least once:
unique visible prefix KV, row q/k/v, W_o, W_lm, drafter logits and the small
per-row outputs; flops of attention over visible keys only, W_o and the LM
head.  Implementation traffic (split-KV partials, the fp32 logits round trip)
is not counted here.
"""
from __future__ import annotations

import numpy as np


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, bytes_per_el: int = 2) -> int:
    """K and V bytes one token adds to a KV cache across `layers` attention
    layers (the per-token KV arithmetic of the Dev.to/aiwithghost DSpine page,
    memory section)."""
    return 2 * layers * kv_heads * head_dim * bytes_per_el


def _elt(dtype: str) -> int:
    return 2 if dtype == "bf16" else 4


def _visible_prefix_tokens(st) -> int:
    """Unique prefix tokens read by the step (shared stems counted once)."""
    spans = sorted(zip(np.asarray(st.root_kv_off).tolist(), np.asarray(st.root_kv_len).tolist()))
    total, cur_lo, cur_hi = 0, None, None
    for off, ln in spans:
        lo, hi = off, off + ln
        if ln == 0:
            continue
        if cur_hi is None or lo > cur_hi:
            if cur_hi is not None:
                total += cur_hi - cur_lo
            cur_lo, cur_hi = lo, hi
        else:
            cur_hi = max(cur_hi, hi)
    if cur_hi is not None:
        total += cur_hi - cur_lo
    return int(total)


def _tree_depths(parent):
    depth = np.zeros(len(parent), np.int64)
    for i, p in enumerate(parent):
        depth[i] = 0 if p < 0 else depth[p] + 1
    return depth


def step_bytes(cfg, st, fp8: bool = False) -> dict:
    """Algorithmic HBM bytes of one step, by stage (`fp8`: the LM head reads
    e4m3 weights, one byte each plus a 4-byte scale per row, and e4m3
    activations)."""
    e = _elt(cfg.dtype)
    n = st.n_rows
    n_draft = int((np.asarray(st.parent) >= 0).sum())
    Hq, Hkv, d, H, V = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.hidden, cfg.vocab
    kv = _visible_prefix_tokens(st) * Hkv * d * e * 2
    rows = n * (Hq + 2 * Hkv) * d * e
    w_o = H * Hq * d * e
    w_lm = V * H + V * 4 if fp8 else V * H * e
    act = n * H * (1 if fp8 else e)
    drafter = n_draft * V * e
    outs = n * 4 * 6 + st.n_roots * 4 * 4
    return {"attention": kv + rows, "w_o": w_o, "lm_head": w_lm + act,
            "drafter": drafter, "outputs": outs,
            "total": kv + rows + w_o + w_lm + drafter + outs}


def step_flops(cfg, st) -> dict:
    """Algorithmic flops of one step (multiply-add = 2), by stage."""
    n = st.n_rows
    Hq, d, H, V = cfg.n_q_heads, cfg.head_dim, cfg.hidden, cfg.vocab
    depth = _tree_depths(np.asarray(st.parent))
    # tree index of every row
    tree = np.cumsum(np.asarray(st.parent) < 0) - 1
    vis = np.asarray(st.root_kv_len)[tree] + depth + 1
    attn = int(vis.sum()) * Hq * d * 2 * 2
    w_o = n * H * Hq * d * 2
    lm = n * V * H * 2
    return {"attention": attn, "w_o": w_o, "lm_head": lm, "total": attn + w_o + lm}
