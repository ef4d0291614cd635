"""Commit step and multi-step chain decoding on the GPU vs the CPU oracle
(through the C ABI; needs an MI355X)."""
import numpy as np
import pytest

from draft_block_verification_verify_amd import workloads as W
from oracle import verify_oracle as O
from tests import parity as P
from tests.test_gpu_parity import MINIS, _record, _say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from draft_block_verification_verify_amd import binding
    binding.lib()
    yield


def _cache_bits(t, dtype):
    import torch
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _compare_caches(dc, kk_o, vv_o, dtype, rep):
    """V bit for bit; K (rotated on each side) within one unit in the last
    place of the cache format, almost always identical."""
    gk, gv = _cache_bits(dc.kv_k, dtype), _cache_bits(dc.kv_v, dtype)
    if dtype == "bf16":
        assert (gv == vv_o).all()
        dk = np.abs(gk.astype(np.int64) - kk_o.astype(np.int64))
    else:
        assert (gv.view(np.int32) == vv_o.view(np.int32)).all()
        dk = np.abs(gk.view(np.int32).astype(np.int64) - kk_o.view(np.int32).astype(np.int64))
    assert dk.max() <= 1, dk.max()
    rep["k_ulp_max"] = max(rep.get("k_ulp_max", 0), int(dk.max()))
    rep["k_not_identical"] = rep.get("k_not_identical", 0) + int((dk > 0).sum())


def run_steps(name, seed, steps):
    from draft_block_verification_verify_amd.runner import DeviceCase
    cfg = MINIS[name]
    gamma = cfg.gamma
    _say(f"[commit] {name} seed={seed} steps={steps}")
    inp = W.make_inputs(cfg, seed, slack=steps * (gamma + 1))
    c = O.cfg_dict(cfg)
    a = dict(O.inp_dict(inp))
    st = inp.st
    n, nd = st.n_rows, int((st.parent >= 0).sum())
    dc = DeviceCase(inp, with_logits=True, max_pos=int(st.pos.max()) + 1 + steps * (gamma + 1))
    kk_o, vv_o = a["kv_k"], a["kv_v"]
    rep = {"walks_from_gpu": 0}
    gpu = dec = None
    try:
        for r in range(steps):
            if r > 0:
                rows = W.round_rows(cfg, seed, r, n, nd)
                dc.next_step(gpu["accept_len"], rows)
                # the oracle's layout follows its own walk (the GPU's only at a near tie)
                parent, pos, off, ln = O.advance(a, dec, gamma)
                assert (dc.inp.st.pos == pos).all() and (dc.inp.st.root_kv_len == ln).all()
                assert (dc.inp.st.parent == parent).all() and (dc.inp.st.root_kv_off == off).all()
                a = dict(a, parent=parent, pos=pos, root_kv_off=off, root_kv_len=ln, **rows)
            a["kv_k"], a["kv_v"] = kk_o, vv_o
            # plant on the oracle's greedy tokens
            W.plant_chain_drafts(dc.inp, O.target_greedy(c, a), rnd=r)
            dc.refresh()
            a["draft_ids"] = dc.inp.draft_ids.copy()
            dc.run()
            gpu = dc.results()
            ref = O.verify(c, a, keep_logits=True)
            P.check_self_consistency(a["parent"], a["draft_ids"], gpu)
            P.compare(ref, gpu, a["parent"], a["draft_ids"], logits_ref=ref["logits"], logits_gpu=gpu["logits"],
                      report=rep)
            dec, from_gpu = P.walk_decisions(ref, gpu, a["parent"])
            rep["walks_from_gpu"] += from_gpu
            dc.commit()
            kk_o, vv_o = O.commit(c, a, dec, kk_o, vv_o)
            _compare_caches(dc, kk_o, vv_o, cfg.dtype, rep)
            rep[f"accept_mean_step{r}"] = float(np.mean(gpu["accept_len"]))
    finally:
        dc.close()
    _record(f"{name}/commit{steps}", rep)
    return rep


@pytest.mark.parametrize("name", ["c1", "c2m", "c5s"])
def test_commit_single_step(name):
    run_steps(name, 0, 1)


@pytest.mark.parametrize("name,steps", [("c2m", 4), ("c5s", 3), ("c1", 3)])
def test_multi_step_chains(name, steps):
    rep = run_steps(name, 1, steps)
    # planted drafts: most steps accept more than the bonus token
    assert max(v for k, v in rep.items() if k.startswith("accept_mean")) > 1.0


def test_commit_refusals():
    import torch
    from draft_block_verification_verify_amd import binding as B
    from draft_block_verification_verify_amd.runner import DeviceCase
    # no slack after the prefix: the accepted path would leave the cache
    cfg = MINIS["c2m"]
    inp = W.make_inputs(cfg, 0)
    dc = DeviceCase(inp)
    try:
        dc.run()
        with pytest.raises(B.SpecVerifyError) as e:
            dc.commit()
        assert e.value.status == B.SV_ERR_BAD_TREE
    finally:
        dc.close()
    # shared stem: every branch's path would overwrite the stem
    inp = W.make_inputs(MINIS["c4m"], 0)
    dc = DeviceCase(inp)
    try:
        dc.run()
        with pytest.raises(B.SpecVerifyError) as e:
            dc.commit()
        assert e.value.status == B.SV_ERR_BAD_TREE
    finally:
        dc.close()
    # inputs or stream other than the last run's
    inp = W.make_inputs(cfg, 0, slack=cfg.gamma + 1)
    dc = DeviceCase(inp)
    try:
        dc.run()
        side = torch.cuda.Stream()
        with pytest.raises(B.SpecVerifyError) as e:
            dc.commit(stream=side.cuda_stream)
        assert e.value.status == B.SV_ERR_INVALID_ARG
        inp.st.root_kv_len = inp.st.root_kv_len + 1
        dc.refresh()
        with pytest.raises(B.SpecVerifyError) as e:
            dc.commit()
        assert e.value.status == B.SV_ERR_INVALID_ARG
        torch.cuda.synchronize()
    finally:
        dc.close()
