"""The T = 1 parity rule (tests/parity.py:check_sample) on the CPU: the
oracle's own outputs pass it, planted mistakes fail it."""
import numpy as np
import pytest

from draft_block_verification_verify_amd import workloads as W
from oracle import verify_oracle as O
from tests import parity as P


def _case(seed):
    inp = W.make_inputs(1, seed)
    W.sample_tree_drafts(inp)
    ua, ub = W.make_uniforms(inp)
    d = dict(O.inp_dict(inp))
    d.update(mode=1, u_accept=ua, u_bonus=ub)
    ref = O.verify(O.cfg_dict(inp.cfg), d, keep_logits=True)
    dl = O.decode(inp.drafter_logits, "f32")
    return inp, ref, ua, ub, dl


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_oracle_outputs_pass(seed):
    inp, ref, ua, ub, dl = _case(seed)
    rep = P.check_sample(inp.st.parent, inp.draft_ids, ua, ub, ref["logits"], dl, ref)
    assert rep["walks"] == 1 and rep["draw_slack"] == 0.0


def test_planted_bonus_outside_its_interval_fails():
    inp, ref, ua, ub, dl = _case(0)
    bad = dict(ref)
    last = int(ref["last_row"][0])
    p = O.softmax(ref["logits"][last])
    # the token farthest from the drawn one in running probability
    cdf = np.cumsum(p)
    far = int(np.argmin(np.abs(cdf - (1.0 - float(ub[0])))))
    if abs(cdf[far] - float(ub[0])) < 0.05:
        far = 0 if float(ub[0]) > 0.5 else len(p) - 1
    bad["bonus"] = np.array([far])
    with pytest.raises(AssertionError):
        P.check_sample(inp.st.parent, inp.draft_ids, ua, ub, ref["logits"], dl, bad)


def test_planted_early_stop_fails_when_the_oracle_clearly_accepts():
    inp, ref, ua, ub, dl = _case(1)
    ua = ua.copy()
    ua[1:] = 0.0                       # every accept test clearly passes
    d = dict(O.inp_dict(inp))
    d.update(mode=1, u_accept=ua, u_bonus=ub)
    ref = O.verify(O.cfg_dict(inp.cfg), d, keep_logits=True)
    assert ref["accept_len"][0] == inp.st.n_rows
    bad = dict(ref)
    bad["accept_len"], bad["last_row"] = np.array([2]), np.array([1])
    with pytest.raises(AssertionError):
        P.check_sample(inp.st.parent, inp.draft_ids, ua, ub, ref["logits"], dl, bad)
