"""The library's verify-budget schedule (host-only C ABI) against the
enumerating oracle.  Runs on the CPU: the call does no GPU work."""
import numpy as np
import pytest

from draft_block_verification_verify_amd import binding as B
from oracle import schedule_oracle as S


def _flat(reqs):
    n = [len(p) for p, _ in reqs]
    par = [x for p, _ in reqs for x in p]
    conf = [x for _, c in reqs for x in c]
    return n, par, conf


def _split(sel, reqs):
    out, o = [], 0
    for p, _ in reqs:
        out.append(tuple(int(x) for x in sel[o:o + len(p)]))
        o += len(p)
    return tuple(out)


def _evaluate(reqs, choice, xs, ys):
    """Expected tokens / ms of a selection, by the oracle's definitions."""
    tok = len(reqs) + sum(float(np.dot(b, S.path_scores(p, c))) for b, (p, c) in zip(choice, reqs))
    return tok, S.step_ms(xs, ys, len(reqs) + sum(sum(b) for b in choice))


def _random_case(r, tree):
    reqs = []
    for _ in range(int(r.integers(1, 4))):
        k = int(r.integers(0, 5))
        par = [int(r.integers(-1, j)) if tree else j - 1 for j in range(k)]
        conf = r.uniform(0, 1, k).astype(np.float32)
        if k and r.random() < 0.3:
            conf[int(r.integers(0, k))] = 1.0
        reqs.append((par, [float(c) for c in conf]))
    npts = int(r.integers(1, 5))
    xs = np.sort(r.choice(np.arange(1, 20), size=npts, replace=False)).tolist()
    ys = np.cumsum(r.uniform(0, 1, npts).astype(np.float32) + np.float32(0.05)).astype(np.float32).tolist()
    return reqs, xs, ys


@pytest.mark.parametrize("tree", [False, True])
def test_matches_enumeration(tree):
    r = np.random.default_rng(7 if tree else 8)
    for _ in range(150):
        reqs, xs, ys = _random_case(r, tree)
        cap = int(r.integers(0, 10)) if r.random() < 0.3 else 0
        if cap and cap < len(reqs):
            cap = len(reqs)
        n, par, conf = _flat(reqs)
        sel, tok, ms = B.spec_verify_schedule(n, par, conf, xs, ys, cap)
        best = S.best_schedule(reqs, xs, ys, cap)
        choice = _split(sel, reqs)
        # the library's selection is closed, within the cap, and optimal
        for b, (p, _) in zip(choice, reqs):
            assert all(not x or p[k] == -1 or b[p[k]] for k, x in enumerate(b))
        rows = len(reqs) + int(sel.sum())
        assert cap == 0 or rows <= cap
        t2, m2 = _evaluate(reqs, choice, xs, ys)
        assert t2 == pytest.approx(tok, rel=1e-9) and m2 == pytest.approx(ms, rel=1e-9)
        assert tok / ms == pytest.approx(best[0], rel=1e-9)


def test_ties_keep_parents():
    # confidence 1 everywhere: all scores equal; any budget keeps prefixes
    reqs = [(list(range(-1, 5)), [1.0] * 6)] * 3
    n, par, conf = _flat(reqs)
    for cap in range(3, 22):
        sel, tok, ms = B.spec_verify_schedule(n, par, conf, [1, 50], [1.0, 1.0], cap)
        for b, (p, _) in zip(_split(sel, reqs), reqs):
            assert all(not x or p[k] == -1 or b[p[k]] for k, x in enumerate(b))
        assert len(reqs) + sel.sum() == cap


def test_large_batch_is_locally_optimal():
    # 32 chains of 7: no single closed add or drop improves tokens / ms
    r = np.random.default_rng(3)
    reqs = []
    for _ in range(32):
        a = r.uniform(0.3, 0.95)
        reqs.append((list(range(-1, 6)), [float(np.float32(a * (1 - 0.03 * j))) for j in range(7)]))
    xs, ys = [32, 64, 128, 192, 256], [0.9, 0.95, 1.05, 1.15, 1.25]
    n, par, conf = _flat(reqs)
    sel, tok, ms = B.spec_verify_schedule(n, par, conf, xs, ys)
    choice = [list(b) for b in _split(sel, reqs)]
    base = tok / ms
    for i, b in enumerate(choice):
        g = sum(b)
        for ng in (g - 1, g + 1):
            if 0 <= ng <= 7:
                alt = [list(x) for x in choice]
                alt[i] = [1] * ng + [0] * (7 - ng)
                t2, m2 = _evaluate(reqs, alt, xs, ys)
                assert t2 / m2 <= base * (1 + 1e-12)


def test_errors():
    with pytest.raises(B.SpecVerifyError) as e:
        B.spec_verify_schedule([2], [-1, 0], [0.5, 1.5], [1], [1.0])
    assert e.value.status == B.SV_ERR_INVALID_ARG
    with pytest.raises(B.SpecVerifyError) as e:
        B.spec_verify_schedule([2], [1, -1], [0.5, 0.5], [1], [1.0])
    assert e.value.status == B.SV_ERR_BAD_TREE
    with pytest.raises(B.SpecVerifyError) as e:
        B.spec_verify_schedule([1], [-1], [0.5], [1, 2], [2.0, 1.0])
    assert e.value.status == B.SV_ERR_INVALID_ARG
    with pytest.raises(B.SpecVerifyError) as e:
        B.spec_verify_schedule([1, 1], [-1, -1], [0.5, 0.5], [1], [1.0], 1)
    assert e.value.status == B.SV_ERR_CAPACITY
