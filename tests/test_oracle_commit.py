"""Pins of the oracle's commit step (step 10) and the next step's layout."""
import numpy as np
import pytest

from draft_block_verification_verify_amd import workloads as W
from oracle import verify_oracle as O


def tiny(kind, dtype="f32", **kw):
    base = dict(cfg_id=91, name="tiny-commit", dtype=dtype, n_q_heads=4, n_kv_heads=2, head_dim=16,
                hidden=32, vocab=300, kind=kind, w_lm_std=0.25)
    base.update(kw)
    return W.Config(**base)


# ---- the cache's number format ---------------------------------------------


def test_bf16_format_hand_values():
    x = [1.0,                  # exact
         1.0 + 2.0 ** -8,      # halfway between 1 and 1 + 2^-7: even mantissa (1.0)
         1.0 + 3 * 2.0 ** -9,  # above halfway: up
         1.0 + 2.0 ** -7 + 2.0 ** -8,   # halfway between odd 1+2^-7 and even 1+2^-6: up to even
         -2.5, 1e-40]
    got = O.to_cache_format(x, "bf16").tolist()
    assert got == [0x3F80, 0x3F80, 0x3F81, 0x3F82, 0xC020, 0x0001]


def test_bf16_format_is_nearest_even():
    # brute force over the two bf16 neighbours of each fp32 value
    r = np.random.default_rng(5)
    f = (r.standard_normal(20000) * np.exp(r.uniform(-20, 20, 20000))).astype(np.float32)
    # add exact halfway cases: low 16 bits 0x8000
    u = f.view(np.uint32)
    f = np.concatenate([f, ((u & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)])
    got = O.to_cache_format(f, "bf16").astype(np.uint32)
    u = f.view(np.uint32)
    lo = u >> 16
    hi = lo + 1
    val = lambda b: (b << 16).view(np.float32).astype(np.float64)
    x = f.astype(np.float64)
    dlo, dhi = np.abs(x - val(lo)), np.abs(x - val(hi))
    want = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    assert (got == want).all()


def test_f32_format_is_the_fp32_value():
    x = np.random.default_rng(1).standard_normal(1000)
    assert (O.to_cache_format(x, "f32") == x.astype(np.float32)).all()


# ---- commit on hand-built layouts -------------------------------------------


def _hand_inputs(dtype="f32"):
    # tree 0: 0 -> {1, 2}, 1 -> 3, 2 -> 4 -> 5 ; tree 1: 6 -> 7 -> 8
    parent = np.array([-1, 0, 0, 1, 2, 4, -1, 6, 7], np.int32)
    pos = np.zeros(9, np.int32)          # position 0: the rotation is the identity
    Hkv, d = 2, 8
    r = np.random.default_rng(3)
    k_rows = r.standard_normal((9, Hkv, d)).astype(np.float32)
    v_rows = r.standard_normal((9, Hkv, d)).astype(np.float32)
    inp = {"parent": parent, "pos": pos, "root_kv_off": np.array([0, 20], np.int64),
           "root_kv_len": np.array([5, 3], np.int32), "k_rows": k_rows, "v_rows": v_rows}
    cfg = {"dtype": dtype, "rope_base": 10000.0}
    kv = r.standard_normal((40, Hkv, d)).astype(np.float32)
    return cfg, inp, kv, kv.copy() + 1


def test_commit_compacts_the_accepted_path():
    cfg, inp, kk0, vv0 = _hand_inputs()
    res = {"accept_len": [4, 2], "last_row": [5, 7]}
    kk, vv = O.commit(cfg, inp, res, kk0, vv0)
    # tree 0: path 0, 2, 4, 5 at entries 5..8; tree 1: path 6, 7 at 23..24
    for dst, row in [(5, 0), (6, 2), (7, 4), (8, 5), (23, 6), (24, 7)]:
        assert (kk[dst] == inp["k_rows"][row]).all()
        assert (vv[dst] == inp["v_rows"][row]).all()
    untouched = [i for i in range(40) if i not in (5, 6, 7, 8, 23, 24)]
    assert (kk[untouched] == kk0[untouched]).all() and (vv[untouched] == vv0[untouched]).all()
    # the caller's arrays are not modified
    assert not np.shares_memory(kk, kk0)


def test_commit_root_only():
    cfg, inp, kk0, vv0 = _hand_inputs()
    kk, vv = O.commit(cfg, inp, {"accept_len": [1, 1], "last_row": [0, 6]}, kk0, vv0)
    assert (kk[5] == inp["k_rows"][0]).all() and (kk[23] == inp["k_rows"][6]).all()
    assert (kk[6] == kk0[6]).all() and (kk[24] == kk0[24]).all()


def test_commit_rejects_inconsistent_results():
    cfg, inp, kk0, vv0 = _hand_inputs()
    with pytest.raises(ValueError):
        O.commit(cfg, inp, {"accept_len": [3, 1], "last_row": [5, 6]}, kk0, vv0)


def test_advance_layout():
    inp = {"parent": np.array([-1, 0, 1, -1, 3, 4], np.int32),
           "pos": np.array([10, 11, 12, 4, 5, 6], np.int32),
           "root_kv_off": np.array([0, 100], np.int64), "root_kv_len": np.array([10, 4], np.int32)}
    parent, pos, off, ln = O.advance(inp, {"accept_len": [3, 1]}, gamma=2)
    assert parent.tolist() == [-1, 0, 1, -1, 3, 4]
    assert pos.tolist() == [13, 14, 15, 5, 6, 7]
    assert off.tolist() == [0, 100] and ln.tolist() == [13, 5]


# ---- committing and continuing equals one longer tree ------------------------


@pytest.mark.parametrize("k_acc", [0, 2, 5])
def test_commit_then_continue_equals_one_tree(k_acc):
    """A row X verified in the next step, after the accepted path was
    committed, attends exactly as X would as a child of the last accepted row
    in the first step's tree (same keys and values, same positions)."""
    gamma = 5
    cfg = tiny("chain", prefix=24, gamma=gamma)
    inp = W.make_inputs(cfg, 2, slack=gamma + 1)
    c, a = O.cfg_dict(cfg), O.inp_dict(inp)
    greedy = O.target_greedy(c, a)
    W.plant_chain_drafts(inp, greedy, k_per_tree=[k_acc])
    a = O.inp_dict(inp)
    res = O.verify(c, a)
    assert res["accept_len"][0] == k_acc + 1
    kk, vv = O.commit(c, a, res, a["kv_k"], a["kv_v"])
    last = int(res["last_row"][0])

    r = np.random.default_rng(9)
    qx = r.standard_normal((1, cfg.n_q_heads, cfg.head_dim)).astype(np.float32)
    kx = r.standard_normal((1, cfg.n_kv_heads, cfg.head_dim)).astype(np.float32)
    vx = r.standard_normal((1, cfg.n_kv_heads, cfg.head_dim)).astype(np.float32)

    # next step: X alone, as the new root
    parent, pos, off, ln = O.advance(a, res, gamma=0)
    nxt = dict(a, parent=parent, pos=pos, root_kv_off=off, root_kv_len=ln, kv_k=kk, kv_v=vv,
               q_rows=qx, k_rows=kx, v_rows=vx)
    o_next = O.attention_outputs(c, nxt, [0])[0]

    # one tree: X as a child of the last accepted row
    n = len(a["parent"])
    one = dict(a, parent=np.append(a["parent"], last).astype(np.int32),
               pos=np.append(a["pos"], a["pos"][last] + 1).astype(np.int32),
               q_rows=np.concatenate([a["q_rows"], qx]), k_rows=np.concatenate([a["k_rows"], kx]),
               v_rows=np.concatenate([a["v_rows"], vx]))
    o_one = O.attention_outputs(c, one, [n])[n]
    assert pos[0] == a["pos"][last] + 1
    np.testing.assert_allclose(o_next, o_one, rtol=1e-5, atol=1e-6)
