"""Pins of the oracle's T = 1 stochastic verification (step 9 of its header).

The rule is pinned by what it must satisfy, not by retyping it: the first
token it emits is distributed exactly as the target p (the defining property
of speculative sampling), its acceptance probability equals the overlap
sum_u min(p, q) = 1 - TV (VESSL 'Speculative Decoding Part 2', DSpark
section), the expected number of accepted drafts of a chain equals the sum
of the prefix survival products (SpecOPD summary, "how it is used"), and
hand-worked cases (tests/golden/stochastic_examples.json).
"""
import json
import os

import numpy as np
import pytest

from oracle import verify_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "stochastic_examples.json")


def _walk(parent, p_rows, q_rows, drafts, u_acc, u_bonus):
    f = O.Forest(np.asarray(parent))
    return O.stochastic_walk(f, 0, lambda i: np.asarray(p_rows[i], float), lambda i: np.asarray(q_rows[i], float),
                             drafts, u_acc, u_bonus)


def test_golden_cases():
    data = json.load(open(GOLDEN))
    for c in data["cases"]:
        q = {int(k): v for k, v in c["q"].items()}
        acc, bonus, last, _ = _walk(c["parent"], c["p"], q, c["draft_ids"], c["u_accept"], c["u_bonus"])
        e = c["expect"]
        assert (acc, bonus, last) == (e["accept_len"], e["bonus"], e["last_row"]), c["name"]


def test_inverse_cdf_skips_zero_weights_and_covers_the_range():
    w = np.array([0.0, 2.0, 0.0, 1.0, 1.0])
    toks = [O.sample_inverse_cdf(w, u)[0] for u in np.linspace(0, 0.999, 400)]
    assert set(toks) == {1, 3, 4}
    assert toks == sorted(toks)                           # monotone in u
    frac = {t: toks.count(t) / len(toks) for t in set(toks)}
    assert abs(frac[1] - 0.5) < 0.01 and abs(frac[3] - 0.25) < 0.01


def _exact_first_token_law(p0, q1, p1, N=2048):
    """Law of the first emitted token of a one-draft chain, integrating the
    oracle's rule over the draft d ~ q1 and over midpoint grids of both
    uniforms."""
    V = len(p0)
    grid = (np.arange(N) + 0.5) / N
    law = np.zeros(V)
    acc_prob = 0.0
    for d in range(V):
        if q1[d] == 0:
            continue
        drafts = [0, d]
        accepted = sum(_walk([-1, 0], [p0, p1], {1: q1}, drafts, [0.0, u], 0.5)[0] == 2 for u in grid) / N
        acc_prob += q1[d] * accepted
        law[d] += q1[d] * accepted
        if accepted < 1.0:
            # a rejection: the emitted token is the bonus draw
            toks = [_walk([-1, 0], [p0, p1], {1: q1}, drafts, [0.0, 1.0 - 1e-12], float(u))[1] for u in grid]
            counts = np.bincount(toks, minlength=V) / N
            law += q1[d] * (1.0 - accepted) * counts
    return law, acc_prob


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_first_token_is_distributed_as_the_target(seed):
    rng = np.random.default_rng(seed)
    V = 5
    p0 = rng.dirichlet(np.ones(V))
    q1 = rng.dirichlet(np.ones(V) * 0.7)
    p1 = rng.dirichlet(np.ones(V))
    law, acc = _exact_first_token_law(p0, q1, p1)
    np.testing.assert_allclose(law, p0, atol=3e-3)
    # acceptance probability = overlap = 1 - TV
    assert abs(acc - O.overlap(p0, q1)) < 2e-3
    assert abs(acc - (1 - 0.5 * np.abs(p0 - q1).sum())) < 2e-3


def test_equal_drafter_always_accepts():
    p = np.array([0.2, 0.3, 0.5])
    for u in np.linspace(0, 0.999, 50):
        for d in range(3):
            acc, _, last, _ = _walk([-1, 0], [p, p], {1: p}, [0, d], [0.0, float(u)], 0.5)
            assert acc == 2 and last == 1


def test_expected_accepts_equal_survival_sum():
    # drafts drawn from the drafter: E[accepted drafts] = sum of prefix survival
    rng = np.random.default_rng(7)
    V, gamma, trials = 6, 3, 20000
    p = [rng.dirichlet(np.ones(V)) for _ in range(gamma + 1)]
    q = {i: rng.dirichlet(np.ones(V)) for i in range(1, gamma + 1)}
    parent = [-1] + list(range(gamma))
    total = 0
    for _ in range(trials):
        drafts = [0] + [int(rng.choice(V, p=q[i])) for i in range(1, gamma + 1)]
        u = [0.0] + list(rng.random(gamma))
        acc, _, _, _ = _walk(parent, p, q, drafts, u, float(rng.random()))
        total += acc - 1
    ov = [1.0] + [O.overlap(p[i - 1], q[i]) for i in range(1, gamma + 1)]
    surv, sums = O.survival(O.Forest(np.asarray(parent)), ov)
    mean = total / trials
    assert abs(mean - sums[0]) < 4 * np.sqrt(gamma * gamma / 4 / trials) + 0.01


def test_branching_nodes_are_refused():
    with pytest.raises(ValueError):
        _walk([-1, 0, 0], [[0.5, 0.5]] * 3, {1: [0.5, 0.5], 2: [0.5, 0.5]}, [0, 0, 1], [0, 0.5, 0.5], 0.5)
