"""Plain CPU oracle of the verify-budget schedule over a batch of requests.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this module.  It shares no code with
the library.

What it computes (VESSL AI "Speculative Decoding Part 2", DSpark section: a
confidence head predicts, per position, the probability that the position
passes given that the earlier ones passed; multiplying these gives the
expected length; the scheduler spends the batch's verify budget on the
positions most likely to pass, across all requests, to maximise throughput on
a measured hardware curve, so gamma varies per request and with load.  Same
page, EAGLE-2: a branch's score is the product of confidences from the root,
so a parent never scores below its child):

1. Request r offers candidate draft positions; candidate k follows parent
   p_k (-1: the request's last committed token, its verify root) and has
   conditional pass probability c_k in [0, 1].  Its score, the probability
   that it is accepted, is the product of c along its path.
2. A selection is a set of candidates containing the parent of each member.
   A request always verifies its root row, so a batch with selection S has
   n_req + |S| rows, and its expected committed tokens are n_req (one bonus
   token per request) + the sum of the scores in S.
3. Step time: the measured curve (rows ascending, ms) interpolated linearly
   between its points, held at its first value below the first point, and
   extended linearly past the last point from its last two points.
4. The schedule maximises expected tokens / step time over all selections
   (with at most max_rows rows when max_rows > 0).  Here: by enumerating
   every selection (tiny cases only).
"""
from __future__ import annotations

import itertools

import numpy as np


def path_scores(parent, conf) -> np.ndarray:
    """Step 1: product of conf along each candidate's path (parents first)."""
    s = np.zeros(len(parent))
    for k, (p, c) in enumerate(zip(parent, conf)):
        if not (p == -1 or 0 <= p < k):
            raise ValueError(f"candidate {k}: parent {p}")
        s[k] = float(c) * (1.0 if p == -1 else s[p])
    return s


def step_ms(curve_rows, curve_ms, rows: float) -> float:
    """Step 3."""
    x = [float(v) for v in curve_rows]
    y = [float(v) for v in curve_ms]
    if rows <= x[0]:
        return y[0]
    for i in range(1, len(x)):
        if rows <= x[i]:
            t = (rows - x[i - 1]) / (x[i] - x[i - 1])
            return y[i - 1] + t * (y[i] - y[i - 1])
    if len(x) == 1:
        return y[0]
    return y[-1] + (rows - x[-1]) * (y[-1] - y[-2]) / (x[-1] - x[-2])


def closed_selections(parent):
    """Every subset of candidates that contains each member's parent."""
    n = len(parent)
    for bits in itertools.product((0, 1), repeat=n):
        if all(not b or parent[k] == -1 or bits[parent[k]] for k, b in enumerate(bits)):
            yield bits


def best_schedule(requests, curve_rows, curve_ms, max_rows: int = 0):
    """Step 4 by enumeration.  `requests`: list of (parent, conf) per request.
    Returns (best value, expected tokens, step ms, selections per request)
    for one maximising selection; values of other maximisers are equal."""
    scores = [path_scores(p, c) for p, c in requests]
    per_req = [list(closed_selections(p)) for p, _ in requests]
    best = None
    for choice in itertools.product(*per_req):
        m = sum(sum(b) for b in choice)
        rows = len(requests) + m
        if max_rows > 0 and rows > max_rows:
            continue
        tok = len(requests) + sum(float(np.dot(b, s)) for b, s in zip(choice, scores))
        ms = step_ms(curve_rows, curve_ms, rows)
        v = tok / ms
        if best is None or v > best[0]:
            best = (v, tok, ms, choice)
    return best
