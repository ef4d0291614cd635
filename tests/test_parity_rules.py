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


# ----------------------------------------------------------------------------
# the greedy-mode rule (tests/parity.py:compare): the oracle's own outputs
# pass, planted mistakes in a copy of them fail
# ----------------------------------------------------------------------------


def _greedy_case(seed=0, w_lm_scale=1.0):
    import dataclasses
    cfg = W.CONFIGS[1]
    if w_lm_scale != 1.0:
        cfg = dataclasses.replace(cfg, cfg_id=91, w_lm_std=cfg.w_lm_std * w_lm_scale)
    inp = W.make_inputs(cfg, seed)
    c = O.cfg_dict(cfg)
    W.plant_chain_drafts(inp, O.target_greedy(c, O.inp_dict(inp)))
    ref = O.verify(c, O.inp_dict(inp), keep_logits=True)
    gpu = {k: np.array(v, copy=True) for k, v in ref.items()}
    return inp, ref, gpu


def test_compare_passes_the_oracle_itself():
    inp, ref, gpu = _greedy_case()
    rep = P.compare(ref, gpu, inp.st.parent, inp.draft_ids, logits_ref=ref["logits"], logits_gpu=gpu["logits"])
    assert rep["lse"] == 0.0 and rep["top_prob"] == 0.0 and rep["prob"] == 0.0


@pytest.mark.parametrize("what", ["lse", "max_peaked", "logit_peaked", "overlap"])
def test_compare_catches_planted_mistakes(what):
    # peaked rows (logit std about 7): the top token's probability is near 1,
    # so a 2e-3 shift of one row's max or top logit moves it past 1e-3
    inp, ref, gpu = _greedy_case(w_lm_scale=5.0 if what != "lse" else 1.0)
    i = 3
    if what == "lse":
        gpu["row_lse"][i] += 1.5e-3                 # past the 1e-3 absolute bound on lse
    elif what == "max_peaked":
        assert np.exp(ref["row_max"][i] - ref["row_lse"][i]) > 0.5
        gpu["row_max"][i] += 2e-3                   # top probability moves by about p_max * 2e-3
    elif what == "logit_peaked":
        top = int(ref["argmax"][i])
        gpu["logits"] = gpu["logits"].copy()
        gpu["logits"][i, top] -= 3e-3
    else:
        gpu["overlap"][i] += 2.5e-3
    with pytest.raises(AssertionError):
        P.compare(ref, gpu, inp.st.parent, inp.draft_ids, logits_ref=ref["logits"], logits_gpu=gpu["logits"])


def test_walk_decisions_take_the_oracle_where_clear():
    inp, ref, gpu = _greedy_case()
    gpu["accept_len"] = gpu["accept_len"] + 0          # same
    dec, from_gpu = P.walk_decisions(ref, gpu, inp.st.parent)
    assert from_gpu == 0 and (dec["accept_len"] == ref["accept_len"]).all()
    ref2 = dict(ref)
    ref2["gap"] = ref["gap"].copy()
    ref2["gap"][int(ref["last_row"][0])] = 1e-4       # a near tie on the walk: the GPU's choice stands
    gpu["accept_len"] = gpu["accept_len"] + 1
    dec, from_gpu = P.walk_decisions(ref2, gpu, inp.st.parent)
    assert from_gpu == 1 and (dec["accept_len"] == gpu["accept_len"]).all()
