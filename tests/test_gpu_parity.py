"""HIP verify step vs the CPU oracle, through the C ABI (needs an MI355X)."""
import dataclasses
import json
import os
import sys

import numpy as np
import pytest

from draft_block_verification_verify_amd import workloads as W
from oracle import verify_oracle as O
from tests import parity as P

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _record(name, rep):
    """Append the worst errors of a parity case to $SV_PARITY_REPORT (jsonl)."""
    path = os.environ.get("SV_PARITY_REPORT")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"case": name, **{k: float(v) for k, v in rep.items()}}) + "\n")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from draft_block_verification_verify_amd import binding
    binding.lib()          # fails loudly if the HIP library is missing
    yield


def mini(base: int, **kw):
    """A small variant of a measured configuration: same head shapes (same
    kernels), smaller hidden / vocab / prefixes, ragged sizes.  The LM-head
    scale keeps the logits' spread near the full configurations' (std about
    1.2-1.4), so the probability rule is tested on distributions of the same
    kind."""
    c = W.CONFIGS[base]
    d = dataclasses.asdict(c)
    d.update(cfg_id=100 + base, name=c.name + "-mini")
    d.update(kw)
    return W.Config(**d)


MINIS = {
    "c1": W.CONFIGS[1],
    "c2m": mini(2, hidden=512, vocab=3001, prefix=301, w_lm_std=0.06),
    "c3m": mini(3, hidden=640, vocab=5000, prefix=777, w_lm_std=0.05),
    "c4m": mini(4, hidden=256, vocab=2048, stem=300, w_lm_std=0.08),
    "c5m": mini(5, hidden=512, vocab=4104, min_len=0, max_len=400, w_lm_std=0.06),
    "c5s": mini(5, hidden=384, vocab=3000, n_seqs=5, min_len=3, max_len=200, w_lm_std=0.06),
    # many tiny trees: attention runs that hold several whole query groups,
    # 768 rows (three 256-row blocks of the blocked activation layouts)
    "c5t": mini(5, hidden=384, vocab=3000, n_seqs=96, min_len=0, max_len=60, w_lm_std=0.06),
    # 96 rows with a vocabulary that is not a multiple of 8 (the tiled LM
    # head's ragged last tile; fp32 logits for the overlap pass)
    "c5v": mini(5, hidden=384, vocab=3001, n_seqs=12, min_len=0, max_len=100, w_lm_std=0.06),
    # 144 rows: one row tile whose 32-row block 4 is partly real (rows 128-143)
    # and whose blocks 5-7 are padding (the waves holding them skip them)
    "c5r": mini(5, hidden=384, vocab=3000, n_seqs=18, min_len=0, max_len=120, w_lm_std=0.06),
    # 17 rows over 240 vocabulary tiles: the small-batch launch with
    # 256-token tiles (fp16 probabilities when no logits buffer is given)
    "c3w": mini(3, hidden=384, vocab=61440, prefix=777, w_lm_std=0.05),
    # 8 rows, 128-token tiles, a vocabulary that is a multiple of 8 (fp16
    # probabilities per 128-token tile without a logits buffer)
    "c2n": mini(2, hidden=512, vocab=3000, prefix=301, w_lm_std=0.06),
}


def run_case(cfg, seed, *, plant=True, with_logits=True, drafter=None, greedy_all=False, fp8=False):
    from draft_block_verification_verify_amd.runner import DeviceCase
    _say(f"[case] {cfg.name} seed={seed} plant={plant} drafter={drafter} fp8={fp8}")
    inp = W.make_inputs(cfg, seed)
    cd, idict = O.cfg_dict(cfg), O.inp_dict(inp)
    if fp8:
        cd["weight_format"] = "fp8"
    if cfg.kind == "tree":
        W.sample_tree_drafts(inp)
    elif plant:
        g = O.target_greedy(cd, idict)
        ks = None
        if greedy_all:
            ks = [cfg.gamma] * inp.st.n_roots
        W.plant_chain_drafts(inp, g, k_per_tree=ks)
    ref0 = None
    if drafter is not None:
        ref0 = O.verify(cd, O.inp_dict(inp), keep_logits=True)
        rng = np.random.default_rng(1234 + seed)
        rows = W.draft_rows(inp.st.parent)
        lg = np.stack([ref0["logits"][inp.st.parent[i]] for i in rows])
        if drafter == "equal":
            q = lg
        else:
            q = lg + rng.standard_normal(lg.shape) * float(drafter)
        q = q.astype(np.float32)
        inp.drafter_logits = W.f32_to_bf16_bits(q) if cfg.dtype == "bf16" else q
    ref = O.verify(cd, O.inp_dict(inp), keep_logits=True)
    dc = DeviceCase(inp, with_logits=with_logits, fp8=fp8)
    dc.run()
    gpu = dc.results()
    dc.close()
    return inp, ref, gpu


@pytest.mark.parametrize("name", list(MINIS))
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_parity_small(name, seed):
    cfg = MINIS[name]
    inp, ref, gpu = run_case(cfg, seed)
    rep = {}
    P.check_self_consistency(inp.st.parent, inp.draft_ids, gpu)
    P.compare(ref, gpu, inp.st.parent, inp.draft_ids, logits_ref=ref["logits"], logits_gpu=gpu["logits"], report=rep)
    _record(f"{name}/seed{seed}", rep)


@pytest.mark.parametrize("name", ["c4m", "c5m", "c5t", "c5v", "c5r", "c2m", "c5s", "c3w", "c2n"])
@pytest.mark.parametrize("seed", [0, 1])
def test_parity_without_logits_buffer(name, seed):
    # No caller logits buffer: above 64 rows the LM head then keeps fp16
    # tile-relative probabilities for the overlap pass instead of fp32 logits
    # (the path the benchmark times); every output is held to the same rules.
    cfg = MINIS[name]
    inp, ref, gpu = run_case(cfg, seed, with_logits=False)
    rep = {}
    P.check_self_consistency(inp.st.parent, inp.draft_ids, gpu)
    P.compare(ref, gpu, inp.st.parent, inp.draft_ids, logits_ref=ref["logits"], report=rep)
    _record(f"{name}/seed{seed}/no-logits", rep)


@pytest.mark.parametrize("name,sigma", [("c5m", 0.6), ("c4m", 0.3)])
def test_overlap_without_logits_buffer_correlated_drafter(name, sigma):
    # overlaps far from zero (a drafter close to the target) on the fp16
    # probability path
    inp, ref, gpu = run_case(MINIS[name], 0, drafter=sigma, with_logits=False)
    rep = {}
    P.compare(ref, gpu, inp.st.parent, inp.draft_ids, logits_ref=ref["logits"], report=rep)
    _record(f"{name}/drafter{sigma}/no-logits", rep)
    rows = [i for i in range(len(inp.st.parent)) if inp.st.parent[i] >= 0]
    assert np.mean(ref["overlap"][rows]) > 0.3


@pytest.mark.parametrize("name,sigma", [("c2m", 0.4), ("c5m", 0.6), ("c4m", 0.3), ("c1", 0.5)])
def test_parity_correlated_drafter(name, sigma):
    # q = target logits + noise: overlaps ~0.8, survival far from zero
    cfg = MINIS[name]
    inp, ref, gpu = run_case(cfg, 0, drafter=sigma)
    rep = {}
    P.compare(ref, gpu, inp.st.parent, inp.draft_ids, logits_ref=ref["logits"], logits_gpu=gpu["logits"], report=rep)
    _record(f"{name}/correlated{sigma}", rep)
    assert np.nanmean(ref["survival"][inp.st.parent >= 0]) > 0.05


@pytest.mark.parametrize("name", ["c1", "c3m"])
def test_drafter_equal_to_target_overlap_near_one(name):
    cfg = MINIS[name]
    inp, ref, gpu = run_case(cfg, 1, drafter="equal")
    rep = {}
    P.compare(ref, gpu, inp.st.parent, inp.draft_ids, logits_ref=ref["logits"], logits_gpu=gpu["logits"], report=rep)
    _record(f"{name}/equal", rep)
    rows = inp.st.parent >= 0
    assert ref["overlap"][rows].min() > 0.97


@pytest.mark.parametrize("name", ["c1", "c2m", "c5m"])
def test_greedy_drafts_fully_accepted(name):
    cfg = MINIS[name]
    inp, ref, gpu = run_case(cfg, 3, greedy_all=True)
    clear = ref["gap"] > P.GAP
    for t, (s, e) in enumerate(P.tree_ranges(list(inp.st.parent))):
        if clear[s:e].all():
            assert gpu["accept_len"][t] == e - s


def test_edge_cases_forest():
    # empty prefixes, single-row trees (no drafts), a branching tree, a
    # 64-row chain, ragged vocabulary (not a multiple of 4 or 8)
    cfg = mini(2, hidden=256, vocab=1003, w_lm_std=0.08)
    rng = np.random.default_rng(7)
    parent, pos, offs, lens = [], [], [], []
    tok = 0

    def add_tree(par_local, L, p0):
        nonlocal tok
        s = len(parent)
        for k, pl in enumerate(par_local):
            parent.append(-1 if pl < 0 else s + pl)
            pos.append(p0 + k)
        offs.append(tok)
        lens.append(L)
        tok += L

    add_tree([-1], 0, 0)                                   # lone root, empty prefix
    add_tree([-1, 0, 0, 1, 1, 2, 5], 70, 70)               # branching tree
    add_tree([-1] + list(range(63)), 33, 33)               # 64-row chain
    add_tree([-1, 0, 1], 0, 5)                             # chain with empty prefix
    add_tree([-1], 129, 129)                               # lone root with prefix
    st = W.Structure(np.array(parent, np.int32), np.array(pos, np.int32), np.array(offs, np.int64),
                     np.array(lens, np.int32), tok)
    inp = W.make_inputs(cfg, 0)
    n, nd = st.n_rows, int((st.parent >= 0).sum())
    inp.st = st
    Hq, Hkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    bf = lambda shape, s=1.0: W.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * s)
    inp.kv_k, inp.kv_v = bf((tok, Hkv, d)), bf((tok, Hkv, d))
    inp.q_rows, inp.k_rows, inp.v_rows = bf((n, Hq, d)), bf((n, Hkv, d)), bf((n, Hkv, d))
    inp.drafter_logits = bf((nd, cfg.vocab), 2.0)
    inp.draft_ids = rng.integers(0, cfg.vocab, n).astype(np.int32)
    cd = O.cfg_dict(cfg)
    g = O.target_greedy(cd, O.inp_dict(inp))
    for i in range(n):           # make many drafts match so the walks go deep
        if parent[i] >= 0 and rng.random() < 0.8:
            inp.draft_ids[i] = g[parent[i]]
    ref = O.verify(cd, O.inp_dict(inp), keep_logits=True)
    from draft_block_verification_verify_amd.runner import DeviceCase
    dc = DeviceCase(inp, with_logits=True)
    dc.run()
    gpu = dc.results()
    dc.close()
    P.check_self_consistency(st.parent, inp.draft_ids, gpu)
    P.compare(ref, gpu, st.parent, inp.draft_ids, logits_ref=ref["logits"], logits_gpu=gpu["logits"])


def test_edge_cases_shared_segment():
    # Trees that read one KV segment (the same offset) become attention packs
    # when their lengths are close: here segment A holds a pack of four trees
    # (lengths 130, 129, 200, 290: branching, chains, lone rows), then a pack
    # of a 10-token tree and a root with an empty prefix (lengths not tile
    # multiples, one zero), a tree on segment B, and a last tree back on A
    # (not consecutive with the first pack: its own).  Head dim 128.
    cfg = mini(2, hidden=256, vocab=1003, w_lm_std=0.08)
    rng = np.random.default_rng(11)
    parent, pos, offs, lens = [], [], [], []

    def add_tree(par_local, off, L):
        s = len(parent)
        for k, pl in enumerate(par_local):
            parent.append(-1 if pl < 0 else s + pl)
            pos.append(L + k)
        offs.append(off)
        lens.append(L)

    add_tree([-1, 0, 0, 1, 1, 2, 5], 0, 130)
    add_tree([-1, 0, 1, 2], 0, 129)
    add_tree([-1] + list(range(6)), 0, 200)
    add_tree([-1, 0, 0], 0, 290)
    add_tree([-1, 0, 1, 2, 3], 0, 10)
    add_tree([-1], 0, 0)
    add_tree([-1, 0, 1, 2, 3, 4], 300, 50)
    add_tree([-1, 0, 0, 2, 2, 4, 4], 0, 140)
    tok = 350
    st = W.Structure(np.array(parent, np.int32), np.array(pos, np.int32), np.array(offs, np.int64),
                     np.array(lens, np.int32), tok)
    inp = W.make_inputs(cfg, 0)
    n, nd = st.n_rows, int((st.parent >= 0).sum())
    inp.st = st
    Hq, Hkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    assert d == 128
    bf = lambda shape, s=1.0: W.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * s)
    inp.kv_k, inp.kv_v = bf((tok, Hkv, d)), bf((tok, Hkv, d))
    inp.q_rows, inp.k_rows, inp.v_rows = bf((n, Hq, d)), bf((n, Hkv, d)), bf((n, Hkv, d))
    inp.drafter_logits = bf((nd, cfg.vocab), 2.0)
    inp.draft_ids = rng.integers(0, cfg.vocab, n).astype(np.int32)
    cd = O.cfg_dict(cfg)
    g = O.target_greedy(cd, O.inp_dict(inp))
    for i in range(n):
        if parent[i] >= 0 and rng.random() < 0.8:
            inp.draft_ids[i] = g[parent[i]]
    ref = O.verify(cd, O.inp_dict(inp), keep_logits=True)
    from draft_block_verification_verify_amd.runner import DeviceCase
    dc = DeviceCase(inp, with_logits=True)
    dc.run()
    gpu = dc.results()
    dc.close()
    P.check_self_consistency(st.parent, inp.draft_ids, gpu)
    rep = {}
    P.compare(ref, gpu, st.parent, inp.draft_ids, logits_ref=ref["logits"], logits_gpu=gpu["logits"], report=rep)
    _record("shared-segment", rep)


@pytest.mark.parametrize("name,scale", [("c2m", 5.0), ("c4m", 5.5), ("c5m", 5.0)])
@pytest.mark.parametrize("with_logits", [True, False])
def test_parity_peaked(name, scale, with_logits):
    # peaked target distributions (logit std about 7, top probabilities near
    # 1): the probability rule and the logsumexp / top-token checks bite, on
    # the fp32-logits path and on the fp16 tile-probability path
    cfg = dataclasses.replace(MINIS[name], cfg_id=MINIS[name].cfg_id + 30, name=name + "-peaked",
                              w_lm_std=MINIS[name].w_lm_std * scale)
    inp, ref, gpu = run_case(cfg, 0, with_logits=with_logits)
    rows = list(range(inp.st.n_rows))
    pmax = np.exp(ref["row_max"] - ref["row_lse"])
    rep = {"p_max_median": float(np.median(pmax)),
           "logit_std": float(np.sqrt(np.mean(ref["logits"] ** 2)))}
    assert rep["p_max_median"] > 0.3, rep
    P.check_self_consistency(inp.st.parent, inp.draft_ids, gpu)
    P.compare(ref, gpu, inp.st.parent, inp.draft_ids, rows=rows, logits_ref=ref["logits"],
              logits_gpu=gpu["logits"] if with_logits else None, report=rep)
    _record(f"{name}/peaked" + ("" if with_logits else "/no-logits"), rep)


@pytest.mark.parametrize("sample", [False, True])
def test_draft_ids_outside_the_vocabulary(sample):
    # ids < 0 or >= V are never accepted (greedy: they equal no greedy token;
    # T = 1: their target probability is 0) and nothing is read for them
    cfg = MINIS["c5s"]
    inp = W.make_inputs(cfg, 4)
    cd = O.cfg_dict(cfg)
    W.plant_chain_drafts(inp, O.target_greedy(cd, O.inp_dict(inp)), k_per_tree=[cfg.gamma] * inp.st.n_roots)
    roots = list(np.nonzero(inp.st.parent < 0)[0])
    bad = [-1, cfg.vocab, 1 << 30, -(1 << 31), cfg.vocab + 7]
    for t, r in enumerate(roots):
        inp.draft_ids[r + 1 + (t % cfg.gamma)] = bad[t % len(bad)]
    from draft_block_verification_verify_amd.runner import DeviceCase
    d = dict(O.inp_dict(inp))
    ua = ub = None
    if sample:
        ua, ub = W.make_uniforms(inp)
        ua[:] = 0.0                                   # every in-vocabulary draft the target can emit passes
        d.update(mode=1, u_accept=ua, u_bonus=ub)
    ref = O.verify(cd, d, keep_logits=True)
    dc = DeviceCase(inp, with_logits=True, uniforms=(ua, ub) if sample else None)
    dc.run()
    gpu = dc.results()
    dc.close()
    for t, r in enumerate(roots):
        stop = r + 1 + (t % cfg.gamma)                # the bad draft's row: never reached
        assert gpu["last_row"][t] < stop and gpu["accept_len"][t] <= stop - r
    P.compare(ref, gpu, inp.st.parent, inp.draft_ids, logits_ref=ref["logits"], logits_gpu=gpu["logits"],
              greedy=not sample)
    if sample:
        dl = O.decode(inp.drafter_logits, cfg.dtype)
        P.check_sample(inp.st.parent, inp.draft_ids, ua, ub, ref["logits"], dl, gpu)
    else:
        P.check_self_consistency(inp.st.parent, inp.draft_ids, gpu)


def test_misaligned_buffers_refused_before_enqueue():
    import torch
    from draft_block_verification_verify_amd import binding as B
    from draft_block_verification_verify_amd.runner import DeviceCase
    cfg = MINIS["c2m"]
    inp = W.make_inputs(cfg, 0)
    dc = DeviceCase(inp)
    try:
        for v in dc.outs.values():
            if v is not None:
                v.fill_(-7)
        good_q = dc.q
        flat = torch.empty(good_q.numel() + 8, dtype=good_q.dtype, device=good_q.device)
        dc.q = flat[1:1 + good_q.numel()].view(good_q.shape)      # 2 bytes off a 16-byte boundary
        dc.refresh()
        with pytest.raises(B.SpecVerifyError) as e:
            dc.run()
        assert e.value.status == B.SV_ERR_INVALID_ARG and "q_rows" in str(e.value)
        dc.q = good_q
        good_bonus = dc.outs["bonus"]
        raw = torch.empty(good_bonus.numel() * 4 + 4, dtype=torch.uint8, device=good_q.device)
        dc.outs["bonus"] = raw[2:].view(torch.int16)                # 2 bytes off a 4-byte boundary
        dc.refresh()
        with pytest.raises(B.SpecVerifyError) as e:
            dc.run()
        assert e.value.status == B.SV_ERR_INVALID_ARG and "bonus" in str(e.value)
        dc.outs["bonus"] = good_bonus
        torch.cuda.synchronize()
        assert (dc.outs["argmax"] == -7).all() and (dc.outs["accept_len"] == -7).all()
        dc.refresh()
        dc.run()                                        # the aligned buffers still run
        assert (dc.results()["argmax"] >= 0).all()
    finally:
        dc.close()


def test_no_draft_rows_and_f32_path():
    # roots only: no drafter logits at all
    cfg = W.CONFIGS[1]
    inp = W.make_inputs(cfg, 5)
    st = W.chain_structure([5, 0, 17], 0)
    inp.st = st
    inp.q_rows, inp.k_rows, inp.v_rows = inp.q_rows[:3], inp.k_rows[:3], inp.v_rows[:3]
    inp.kv_k, inp.kv_v = inp.kv_k[:22], inp.kv_v[:22]
    inp.drafter_logits = inp.drafter_logits[:0]
    inp.draft_ids = np.zeros(3, np.int32)
    ref = O.verify(O.cfg_dict(cfg), O.inp_dict(inp), keep_logits=True)
    from draft_block_verification_verify_amd.runner import DeviceCase
    dc = DeviceCase(inp, with_logits=True)
    dc.run()
    gpu = dc.results()
    dc.close()
    P.compare(ref, gpu, st.parent, inp.draft_ids, logits_ref=ref["logits"], logits_gpu=gpu["logits"])
    assert gpu["accept_len"].tolist() == [1, 1, 1]


def test_repeat_runs_bit_identical_and_handle_reuse():
    from draft_block_verification_verify_amd.runner import DeviceCase
    cfg = MINIS["c5m"]
    inp = W.make_inputs(cfg, 4)
    inp.draft_ids = np.random.default_rng(0).integers(0, cfg.vocab, inp.st.n_rows).astype(np.int32)
    dc = DeviceCase(inp, with_logits=True)
    dc.run()
    a = dc.results()
    dc.run()
    b = dc.results()
    for k in a:
        if a[k] is not None:
            np.testing.assert_array_equal(a[k], b[k], err_msg=k)
    # same handle, a smaller second workload (4 of the 32 sequences)
    small = W.make_inputs(cfg, 4)
    rows = np.arange(0, 4 * 8)
    small.st = W.chain_structure(inp.st.root_kv_len[:4], cfg.gamma)
    tok = int(inp.st.root_kv_len[:4].sum())
    small.kv_k, small.kv_v = inp.kv_k[:tok], inp.kv_v[:tok]
    small.q_rows, small.k_rows, small.v_rows = inp.q_rows[rows], inp.k_rows[rows], inp.v_rows[rows]
    small.drafter_logits = inp.drafter_logits[:4 * 7]
    small.draft_ids = inp.draft_ids[rows]
    dc2 = DeviceCase(small, with_logits=True, verifier=dc.ver, weights=(dc.w_o, dc.w_lm))
    dc2.run()
    c = dc2.results()
    # 32 rows take the skinny projection path (256 took the tiled one): check
    # the second run against the oracle
    ref = O.verify(O.cfg_dict(cfg), O.inp_dict(small), keep_logits=True)
    P.check_self_consistency(small.st.parent, small.draft_ids, c)
    P.compare(ref, c, small.st.parent, small.draft_ids, logits_ref=ref["logits"], logits_gpu=c["logits"])
    dc.close()


def test_error_paths_enqueue_nothing():
    import torch
    from draft_block_verification_verify_amd import binding as B
    from draft_block_verification_verify_amd.runner import DeviceCase
    cfg = W.CONFIGS[1]
    inp = W.make_inputs(cfg, 0)
    dc = DeviceCase(inp)
    for v in dc.outs.values():
        if v is not None:
            v.fill_(-7)
    good = inp.st.parent.copy()
    bad = good.copy()
    bad[3] = 5                    # parent after the child
    inp.st.parent = bad
    dc.refresh()
    with pytest.raises(B.SpecVerifyError) as e:
        dc.run()
    assert e.value.status == B.SV_ERR_BAD_TREE
    torch.cuda.synchronize()
    assert (dc.outs["argmax"] == -7).all()
    inp.st.parent = good
    inp.st.pos = inp.st.pos + (1 << 20)        # beyond max_pos
    dc.refresh()
    with pytest.raises(B.SpecVerifyError) as e:
        dc.run()
    assert e.value.status == B.SV_ERR_BAD_TREE
    dc.close()


# ----------------------------------------------------------------------------
# T = 1 stochastic verification (chains)
# ----------------------------------------------------------------------------


def run_sample_case(cfg, seed, sigma=None, with_logits=True):
    """Drafts drawn from the drafter (optionally a drafter correlated with the
    target: its logits = the target's + N(0, sigma)), seeded uniforms."""
    from draft_block_verification_verify_amd.runner import DeviceCase
    _say(f"[sample case] {cfg.name} seed={seed} sigma={sigma}")
    inp = W.make_inputs(cfg, seed)
    cd = O.cfg_dict(cfg)
    if sigma is not None:
        ref0 = O.verify(cd, O.inp_dict(inp), keep_logits=True)
        rows = W.draft_rows(inp.st.parent)
        lg = np.stack([ref0["logits"][inp.st.parent[i]] for i in rows])
        rng = np.random.default_rng(4321 + seed)
        q = (lg + rng.standard_normal(lg.shape) * float(sigma)).astype(np.float32)
        inp.drafter_logits = W.f32_to_bf16_bits(q) if cfg.dtype == "bf16" else q
    W.sample_tree_drafts(inp)
    ua, ub = W.make_uniforms(inp)
    d = dict(O.inp_dict(inp))
    d.update(mode=1, u_accept=ua, u_bonus=ub)
    ref = O.verify(cd, d, keep_logits=True)
    dc = DeviceCase(inp, with_logits=with_logits, uniforms=(ua, ub))
    dc.run()
    gpu = dc.results()
    dc.close()
    return inp, ref, gpu, ua, ub


@pytest.mark.parametrize("name,sigma", [("c1", None), ("c2m", None), ("c3m", 0.4), ("c4m", 0.3),
                                        ("c5m", 0.5), ("c5s", 0.8), ("c1", 0.3)])
def test_parity_sample_mode(name, sigma):
    cfg = MINIS[name]
    inp, ref, gpu, ua, ub = run_sample_case(cfg, 0, sigma)
    st = inp.st
    P.check_self_consistency(st.parent, inp.draft_ids, gpu, greedy=False)
    rep = {}
    P.compare(ref, gpu, st.parent, inp.draft_ids, logits_ref=ref["logits"], logits_gpu=gpu["logits"], report=rep,
              greedy=False)
    dl = O.decode(inp.drafter_logits, cfg.dtype)
    rs = P.check_sample(st.parent, inp.draft_ids, ua, ub, ref["logits"], dl, gpu)
    same = sum(int((gpu["accept_len"][t], gpu["bonus"][t], gpu["last_row"][t]) ==
                   (ref["accept_len"][t], ref["bonus"][t], ref["last_row"][t])) for t in range(st.n_roots))
    rep.update(rs)
    rep["same_as_oracle"] = same / st.n_roots
    _record(f"{name}/sample{sigma}", rep)


@pytest.mark.parametrize("name,sigma", [("c5m", 0.5), ("c4m", 0.3), ("c5t", 0.4), ("c5m", None), ("c5s", 0.5),
                                        ("c3w", 0.4), ("c2n", None)])
def test_parity_sample_mode_without_logits_buffer(name, sigma):
    # above 64 rows without a caller logits buffer the accept tests and the
    # bonus draw read the LM head's fp16 tile-relative probabilities
    cfg = MINIS[name]
    inp, ref, gpu, ua, ub = run_sample_case(cfg, 1, sigma, with_logits=False)
    st = inp.st
    P.check_self_consistency(st.parent, inp.draft_ids, gpu, greedy=False)
    rep = {}
    P.compare(ref, gpu, st.parent, inp.draft_ids, logits_ref=ref["logits"], report=rep, greedy=False)
    dl = O.decode(inp.drafter_logits, cfg.dtype)
    rs = P.check_sample(st.parent, inp.draft_ids, ua, ub, ref["logits"], dl, gpu)
    rep.update(rs)
    _record(f"{name}/sample{sigma}/no-logits", rep)


def test_sample_mode_refuses_branching_and_bad_mode():
    import torch
    from draft_block_verification_verify_amd import binding as B
    from draft_block_verification_verify_amd.runner import DeviceCase
    cfg = W.CONFIGS[1]
    inp = W.make_inputs(cfg, 0)
    ua, ub = W.make_uniforms(inp)
    dc = DeviceCase(inp, uniforms=(ua, ub))
    for v in dc.outs.values():
        if v is not None:
            v.fill_(-7)
    par = inp.st.parent.copy()
    par[3] = 1                      # rows 2 and 3 both children of row 1
    inp.st.parent = par
    dc.refresh()
    with pytest.raises(B.SpecVerifyError) as e:
        dc.run()
    assert e.value.status == B.SV_ERR_UNSUPPORTED
    dc.sv_in.mode = 5
    with pytest.raises(B.SpecVerifyError) as e:
        dc.run()
    assert e.value.status == B.SV_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert (dc.outs["accept_len"] == -7).all()
    dc.close()


# ----------------------------------------------------------------------------
# full sizes, in the bench's launch configuration, on sampled trees
# ----------------------------------------------------------------------------


_FULL = {}


def _full_case(cfg_id, seed):
    """Inputs and oracle outputs of a full-size workload on 8 sampled trees
    (chains: drafts planted on the oracle's greedy tokens of those trees),
    kept for the next case of the same workload and seed."""
    key = (cfg_id, seed)
    if key not in _FULL:
        _FULL.clear()                     # one full-size workload in memory at a time
        cfg = W.CONFIGS[cfg_id]
        _say(f"[full] generating {cfg.name} seed {seed}")
        inp = W.make_inputs(cfg, seed)
        st = inp.st
        trees = P.sampled_trees(st)
        cd = O.cfg_dict(cfg)
        _say(f"[full] oracle on trees {trees}")
        if cfg.kind == "tree":
            W.sample_tree_drafts(inp)
        else:
            g = O.target_greedy(cd, O.inp_dict(inp), trees=trees)
            # planted drafts on the sampled trees; random drafts elsewhere
            W.plant_chain_drafts(inp, np.where(g < 0, 0, g))
        ref = O.verify(cd, O.inp_dict(inp), trees=trees, keep_logits=True)
        _FULL[key] = (inp, ref, trees)
    return _FULL[key]


@pytest.mark.slow
@pytest.mark.parametrize("cfg_id,seed,with_logits", [
    (2, 0, True), (2, 1, True), (2, 2, True), (2, 0, False),
    (3, 0, True), (3, 1, True), (3, 2, True), (3, 0, False),
    # the tree and 32-chain workloads in the benchmark's launch configuration
    # (no logits buffer: fp16 tile probabilities), and once with fp32 logits
    # compared element-wise
    (4, 0, False), (4, 0, True), (4, 1, False), (4, 2, False),
    (5, 0, False), (5, 0, True), (5, 1, False), (5, 2, False),
])
def test_parity_full_size_sampled(cfg_id, seed, with_logits):
    from draft_block_verification_verify_amd.runner import DeviceCase
    inp, ref, trees = _full_case(cfg_id, seed)
    st = inp.st
    _say(f"[full] gpu run (logits buffer: {with_logits})")
    dc = DeviceCase(inp, with_logits=with_logits)
    dc.run()
    gpu = dc.results()
    dc.close()
    P.check_self_consistency(st.parent, inp.draft_ids, gpu)
    rows = [int(i) for i in ref["rows"]]
    rep = {}
    P.compare(ref, gpu, st.parent, inp.draft_ids, rows=rows, logits_ref=ref["logits"],
              logits_gpu=gpu["logits"] if with_logits else None, report=rep)
    rep["trees"] = len(trees)
    rep["rows"] = len(rows)
    _record(f"{inp.cfg.name}/full-sampled/seed{seed}" + ("" if with_logits else "/no-logits"), rep)
    if cfg_id == 5:
        assert int(np.argmax(st.root_kv_len)) in trees        # the longest prefix is scored


@pytest.mark.parametrize("seed", [0, 1])
def test_parity_ragged_gamma(seed):
    # per-sequence draft counts, zero included (what a verify-budget schedule
    # produces); fresh rows on the same prefixes
    from draft_block_verification_verify_amd.runner import DeviceCase
    cfg = MINIS["c5m"]
    base = W.make_inputs(cfg, seed)
    lens = base.st.root_kv_len
    r = np.random.default_rng(50 + seed)
    gam = r.integers(0, cfg.gamma + 1, size=len(lens))
    gam[0] = 0
    st = W.chain_structure(lens, gam)
    n, nd = st.n_rows, int((st.parent >= 0).sum())
    rows = W.round_rows(cfg, seed, 1, n, nd)
    inp = dataclasses.replace(base, st=st, q_rows=rows["q_rows"], k_rows=rows["k_rows"], v_rows=rows["v_rows"],
                              drafter_logits=rows["drafter_logits"], draft_ids=np.zeros(n, np.int32))
    _say(f"[case] ragged gamma seed={seed} rows={n}")
    cd = O.cfg_dict(cfg)
    W.plant_chain_drafts(inp, O.target_greedy(cd, O.inp_dict(inp)))
    ref = O.verify(cd, O.inp_dict(inp), keep_logits=True)
    dc = DeviceCase(inp, with_logits=True)
    try:
        dc.run()
        gpu = dc.results()
    finally:
        dc.close()
    rep = {}
    P.check_self_consistency(st.parent, inp.draft_ids, gpu)
    P.compare(ref, gpu, st.parent, inp.draft_ids, logits_ref=ref["logits"], logits_gpu=gpu["logits"], report=rep)
    _record(f"ragged/seed{seed}", rep)
