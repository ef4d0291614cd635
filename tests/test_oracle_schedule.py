"""Pins of the verify-budget schedule oracle."""
import numpy as np
import pytest

from oracle import schedule_oracle as S


def chain(conf):
    return (list(range(-1, len(conf) - 1)), list(conf))


def test_chain_scores_are_powers():
    a = 0.8
    s = S.path_scores(*chain([a] * 6))
    np.testing.assert_allclose(s, a ** np.arange(1, 7), rtol=1e-15)


def test_tree_scores_multiply_along_paths():
    # 0 <- root, 1 <- 0, 2 <- 0, 3 <- 2
    s = S.path_scores([-1, 0, 0, 2], [0.5, 0.4, 0.9, 0.1])
    np.testing.assert_allclose(s, [0.5, 0.2, 0.45, 0.045], rtol=1e-15)
    with pytest.raises(ValueError):
        S.path_scores([1, -1], [0.5, 0.5])


def test_compounding_of_an_overestimate():
    # the pages: 10 % too high at every position -> about 95 % too high at gamma = 7
    conf = np.full(7, 0.6)
    ratio = S.path_scores(*chain(conf * 1.1))[-1] / S.path_scores(*chain(conf))[-1]
    assert ratio == pytest.approx(1.1 ** 7) and 1.9 < ratio < 2.0


def test_step_time_interpolation():
    xs, ys = [2, 4, 8], [1.0, 2.0, 2.5]
    assert S.step_ms(xs, ys, 1) == 1.0          # held below the first point
    assert S.step_ms(xs, ys, 3) == 1.5
    assert S.step_ms(xs, ys, 6) == 2.25
    assert S.step_ms(xs, ys, 8) == 2.5
    assert S.step_ms(xs, ys, 12) == 3.0         # extended from the last two points


def test_flat_curve_takes_everything():
    # constant step time: the expected length 1 + sum a^j of the whole chain
    a, g = 0.7, 5
    v, tok, ms, sel = S.best_schedule([chain([a] * g)], [1, 100], [2.0, 2.0])
    assert sel == ((1,) * g,)
    assert tok == pytest.approx(1 + a * (1 - a ** g) / (1 - a))
    assert v == pytest.approx(tok / 2.0)


def test_hand_solved_choices():
    req = [chain([0.9, 0.5])]
    # time proportional to rows: one row per token is best (1 token / 1 ms)
    v, tok, ms, sel = S.best_schedule(req, [1, 2, 3], [1.0, 2.0, 3.0])
    assert sel == ((0, 0),) and v == pytest.approx(1.0)
    # fixed cost 1 ms + 0.1 ms per row: verify both (2.35 tokens / 1.3 ms)
    v, tok, ms, sel = S.best_schedule(req, [1, 2, 3], [1.1, 1.2, 1.3])
    assert sel == ((1, 1),) and tok == pytest.approx(2.35) and v == pytest.approx(2.35 / 1.3)


def test_budget_goes_to_the_likelier_request():
    # two requests, room for one draft row: the 0.9 candidate wins
    reqs = [chain([0.3]), chain([0.9])]
    v, tok, ms, sel = S.best_schedule(reqs, [2, 3, 4], [1.0, 1.0, 1.0], max_rows=3)
    assert sel == ((0,), (1,)) and tok == pytest.approx(2.9)


def test_tree_selection_is_closed():
    reqs = [([-1, 0, -1], [0.9, 0.9, 0.2])]
    for bits in S.closed_selections(reqs[0][0]):
        assert not (bits[1] and not bits[0])
    # 0.2 ms fixed + 0.1 ms per row: 2.71 tokens / 0.5 ms beats 2.91 / 0.6
    v, tok, ms, sel = S.best_schedule(reqs, [1, 4], [0.3, 0.6])
    assert sel == ((1, 1, 0),) and v == pytest.approx(2.71 / 0.5)
    # 1.5 ms fixed: the 0.2 branch adds more than the batch's average rate
    v, tok, ms, sel = S.best_schedule(reqs, [1, 4], [1.6, 1.9])
    assert sel == ((1, 1, 1),) and v == pytest.approx(2.91 / 1.9)
