"""FP8 (e4m3, W8A8) LM head of the HIP verify step against the oracle's FP8
head, through the C ABI (needs an MI355X).

Two kinds of case:

* exact activations: every row's normalised hidden state is +-1 on both sides
  (keys 0, so each row attends uniformly to its tree's rows, which share one
  value vector of +-1 entries; W_o a signed permutation with +-1 entries;
  norm epsilon 0), so both sides quantise identical activations and the FP8
  logits differ only by fp32 accumulation: held to 1e-4 of max(|ref|, rms)
  with no flip bound, and every decision exact where the oracle's top-2 gap
  exceeds 1e-2.  This also pins the e4m3 codes of every weight the GPU
  multiplies;
* seeded random inputs with planted top-1 margins (tests/parity.py,
  plant_fp8_margins): the flip bound of the module docstring there still
  applies, and at least 90 % of the rows must have their decision held
  exactly (reported as `clear_fraction`).
"""
import dataclasses

import numpy as np
import pytest

from draft_block_verification_verify_amd import workloads as W
from oracle import verify_oracle as O
from tests import parity as P
from tests.test_gpu_parity import MINIS, _record, _say, mini

pytestmark = pytest.mark.gpu

EXACT_TOL = {"gap": 1e-2, "logit_rel": 1e-4, "prob_abs": 1e-3}

FP8_MINIS = {
    "c2m": MINIS["c2m"],
    "c3m": MINIS["c3m"],
    "c5m": MINIS["c5m"],
    "c5s": MINIS["c5s"],
    # the tree shape with a hidden width above its 448 rows (the margin
    # planting needs no more rows than the hidden width)
    "c4m8": mini(4, hidden=1024, vocab=2048, stem=300, w_lm_std=0.04),
    # 96 rows: above 64 (fp16 probabilities without a logits buffer) and
    # below 128 (the kernel's variant that skips padding rows)
    "c5h": mini(5, hidden=384, vocab=3000, n_seqs=12, min_len=3, max_len=200, w_lm_std=0.06),
    # 96 rows, a vocabulary that is not a multiple of 8: fp32 logits for the
    # overlap pass even without a caller buffer
    "c5v": MINIS["c5v"],
    # 144 rows: the dense kernel with a partly real row block and padding
    # blocks skipped
    "c5r": MINIS["c5r"],
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from draft_block_verification_verify_amd import binding
    binding.lib()          # fails loudly if the HIP library is missing
    yield


def _run(inp, fp8=True, with_logits=True):
    from draft_block_verification_verify_amd.runner import DeviceCase
    dc = DeviceCase(inp, with_logits=with_logits, fp8=fp8)
    try:
        dc.run()
        return dc.results()
    finally:
        dc.close()


def _plant_drafts(inp, greedy, rng, p_match=0.75):
    """Each draft row carries its parent's greedy token with probability
    p_match, else a random token: walks of every depth, branching included."""
    ids = np.zeros(inp.st.n_rows, np.int32)
    for i, p in enumerate(inp.st.parent):
        if p >= 0:
            ids[i] = int(greedy[p]) if rng.random() < p_match else int(rng.integers(0, inp.cfg.vocab))
    inp.draft_ids = ids


# ----------------------------------------------------------------------------
# exact activations
# ----------------------------------------------------------------------------


def exact_activation_inputs(cfg, n_trees, seed):
    rng = np.random.default_rng([seed, 31])
    Hq, Hkv, d, H = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.hidden
    assert H <= Hq * d and cfg.norm_eps == 0.0
    parent, pos, vals = [], [], []
    for _ in range(n_trees):
        nt = int(rng.integers(1, 9))
        s = len(parent)
        v_tree = rng.choice([-1.0, 1.0], size=(Hkv, d)).astype(np.float32)
        for j in range(nt):
            parent.append(-1 if j == 0 else s + int(rng.integers(0, j)))
            pos.append(j)
            vals.append(v_tree)
    n, R = len(parent), n_trees
    kv = 16                                     # a small cache no tree reads (every prefix is empty)
    st = W.Structure(np.array(parent, np.int32), np.array(pos, np.int32), np.zeros(R, np.int64),
                     np.zeros(R, np.int32), kv)
    inp = W.make_inputs(cfg, seed)
    bf = W.f32_to_bf16_bits
    inp.st = st
    inp.kv_k = bf(rng.standard_normal((kv, Hkv, d)).astype(np.float32))
    inp.kv_v = bf(rng.standard_normal((kv, Hkv, d)).astype(np.float32))
    inp.q_rows = bf(rng.standard_normal((n, Hq, d)).astype(np.float32))
    inp.k_rows = bf(np.zeros((n, Hkv, d), np.float32))
    inp.v_rows = bf(np.stack(vals))
    w_o = np.zeros((H, Hq * d), np.float32)
    cols = rng.permutation(Hq * d)[:H]
    w_o[np.arange(H), cols] = rng.choice([-1.0, 1.0], size=H)
    inp.w_o = bf(w_o)
    nd = int((st.parent >= 0).sum())
    inp.drafter_logits = bf((rng.standard_normal((nd, cfg.vocab)) * 2.0).astype(np.float32))
    inp.draft_ids = np.zeros(n, np.int32)
    return inp


@pytest.mark.parametrize("base,n_trees", [("c2m", 10), ("c5m", 70), ("c2m", 90)])
def test_fp8_exact_activations(base, n_trees):
    cfg = dataclasses.replace(MINIS[base], cfg_id=MINIS[base].cfg_id + 50, name=base + "-exact", norm_eps=0.0)
    inp = exact_activation_inputs(cfg, n_trees, seed=n_trees)
    _say(f"[fp8 exact] {cfg.name} trees={n_trees} rows={inp.st.n_rows}")
    cd = dict(O.cfg_dict(cfg), weight_format="fp8")
    # the premise: every oracle hidden row is +-1, so both sides quantise it alike
    hs = O.hidden_states(cd, O.inp_dict(inp), range(inp.st.n_rows))
    assert all(np.array_equal(np.abs(h), np.ones_like(h)) for h in hs.values())
    g = O.target_greedy(cd, O.inp_dict(inp))
    _plant_drafts(inp, g, np.random.default_rng(n_trees))
    ref = O.verify(cd, O.inp_dict(inp), keep_logits=True)
    gpu = _run(inp)
    P.check_self_consistency(inp.st.parent, inp.draft_ids, gpu)
    rep = {}
    P.compare(ref, gpu, inp.st.parent, inp.draft_ids, logits_ref=ref["logits"], logits_gpu=gpu["logits"],
              report=rep, tol=EXACT_TOL)
    n = inp.st.n_rows
    rep["clear_fraction"] = float((ref["gap"] > EXACT_TOL["gap"]).mean())
    rep["accept_len_mean"] = float(gpu["accept_len"].mean())
    _record(f"{cfg.name}/fp8-exact/trees{n_trees}", rep)
    assert rep["clear_fraction"] >= 0.9, rep
    assert (gpu["accept_len"] > 1).any()          # the walks do go deep
    assert n == len(gpu["argmax"])


# ----------------------------------------------------------------------------
# random inputs, planted margins
# ----------------------------------------------------------------------------


def fp8_case(cfg, seed, *, plant=True, with_logits=True):
    _say(f"[fp8] {cfg.name} seed={seed} plant={plant}")
    inp = W.make_inputs(cfg, seed)
    cd = dict(O.cfg_dict(cfg), weight_format="fp8")
    rows = list(range(inp.st.n_rows))
    if plant:
        P.plant_fp8_margins(cd, inp, rows, seed=seed)
    if cfg.kind == "tree":
        W.sample_tree_drafts(inp)
    else:
        W.plant_chain_drafts(inp, O.target_greedy(cd, O.inp_dict(inp)))
    ref = O.verify(cd, O.inp_dict(inp), keep_logits=True)
    gpu = _run(inp, with_logits=with_logits)
    return inp, cd, ref, gpu, rows


def _check_fp8(inp, cd, ref, gpu, rows, name, min_clear):
    P.check_self_consistency(inp.st.parent, inp.draft_ids, gpu)
    alt = P.fp8_alternatives(cd, O.inp_dict(inp), rows)
    bound = P.fp8_bounds(cd, O.inp_dict(inp), rows)
    rep = {}
    P.compare(ref, gpu, inp.st.parent, inp.draft_ids, rows=rows, logits_ref=ref["logits"],
              logits_gpu=gpu["logits"], report=rep, tol=P.FP8_TOL, alt=alt, bound=bound)
    rms = {i: np.sqrt(np.mean(ref["logits"][i] ** 2)) for i in rows}
    rep["flip_bound_max_rel"] = max(float(bound[i].max() / rms[i]) for i in rows)
    rep["clear_fraction"] = P.fp8_clear_fraction(ref, rows, bound, alt)
    _record(name, rep)
    assert rep["clear_fraction"] >= min_clear, rep
    return rep


@pytest.mark.parametrize("name", list(FP8_MINIS))
@pytest.mark.parametrize("seed", [0, 1])
def test_parity_fp8(name, seed):
    inp, cd, ref, gpu, rows = fp8_case(FP8_MINIS[name], seed)
    _check_fp8(inp, cd, ref, gpu, rows, f"{name}/fp8/seed{seed}", 0.9)


@pytest.mark.parametrize("name", ["c5m", "c4m8", "c5h", "c5v", "c5s", "c3m"])
def test_parity_fp8_without_logits_buffer(name):
    # No caller logits buffer: above 64 rows the FP8 LM head then keeps fp16
    # tile-relative probabilities for the overlap pass instead of fp32 logits
    # (the path the benchmark times); every output is held to the same rules.
    inp, cd, ref, gpu, rows = fp8_case(FP8_MINIS[name], 0, with_logits=False)
    assert gpu["logits"] is None
    _check_fp8(inp, cd, ref, gpu, rows, f"{name}/fp8/no-logits", 0.9)


@pytest.mark.parametrize("name", ["c5m", "c5h"])
def test_fp8_logits_buffer_changes_no_decision(name):
    # the same FP8 run with and without a logits buffer: the tile statistics
    # come from the same code either way, so every decision and row
    # statistic is identical; only the overlaps' inputs differ (fp32 logits
    # or fp16 probabilities relative to each tile's maximum, 2^-11 relative)
    inp, cd, ref, with_buf, rows = fp8_case(FP8_MINIS[name], 1)
    without = _run(inp, with_logits=False)
    for k in ("argmax", "accept_len", "bonus", "last_row", "row_max", "row_lse"):
        np.testing.assert_array_equal(without[k], with_buf[k], err_msg=k)
    np.testing.assert_allclose(without["overlap"], with_buf["overlap"], rtol=0, atol=2e-3)
    np.testing.assert_allclose(without["survival"], with_buf["survival"], rtol=0, atol=2e-3)


@pytest.mark.parametrize("name", ["c5m", "c4m8"])
def test_parity_fp8_unplanted(name):
    # unplanted random inputs: most decisions fall inside the flip bound, the
    # rest of the rules (bounded logits, near-maximal choices, self-consistent
    # walks, overlaps) still hold
    inp, cd, ref, gpu, rows = fp8_case(FP8_MINIS[name], 2, plant=False)
    _check_fp8(inp, cd, ref, gpu, rows, f"{name}/fp8/unplanted", 0.0)


@pytest.mark.slow
@pytest.mark.parametrize("with_logits", [True, False])
def test_parity_fp8_full_size_sampled(with_logits):
    # without a logits buffer: the fp16 probability path the benchmark times
    from draft_block_verification_verify_amd.runner import DeviceCase
    cfg = W.CONFIGS[5]
    _say(f"[full fp8] generating {cfg.name}")
    inp = W.make_inputs(cfg, 0)
    st = inp.st
    trees = P.sampled_trees(st)
    cd = dict(O.cfg_dict(cfg), weight_format="fp8")
    roots = list(np.nonzero(st.parent < 0)[0]) + [st.n_rows]
    rows = [i for t in trees for i in range(roots[t], roots[t + 1])]
    _say(f"[full fp8] planting margins on trees {trees} ({len(rows)} rows)")
    P.plant_fp8_margins(cd, inp, rows, seed=0)
    g = O.target_greedy(cd, O.inp_dict(inp), trees=trees)
    W.plant_chain_drafts(inp, np.where(g < 0, 0, g))
    ref = O.verify(cd, O.inp_dict(inp), trees=trees, keep_logits=True)
    _say(f"[full fp8] gpu run, logits buffer {with_logits}")
    dc = DeviceCase(inp, with_logits=with_logits, fp8=True)
    dc.run()
    gpu = dc.results()
    dc.close()
    name = f"{cfg.name}/fp8/full-sampled" + ("" if with_logits else "/no-logits")
    rep = _check_fp8(inp, cd, ref, gpu, [int(i) for i in ref["rows"]], name, 0.9)
    _say(f"[full fp8] clear fraction {rep['clear_fraction']:.3f}")
