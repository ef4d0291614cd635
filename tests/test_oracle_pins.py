"""Pins of the CPU oracle to things other than itself: independent library
routines (torch SDPA), closed forms, constructed special cases, brute force on
tiny inputs and the worked numbers printed on the pages (tests/golden/)."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import verify_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------
# rotary positions
# ----------------------------------------------------------------------------


def test_rope_identity_at_zero_and_norm_preserved():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 64))
    assert np.array_equal(O.rope(x, 0, 10000.0), x)
    for p in (1, 17, 4096, 16400):
        y = O.rope(x, p, 10000.0)
        np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)


def test_rope_relative_position_identity():
    # <R(m) q, R(n) k> depends on m - n only
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    for m, n in [(5, 3), (4100, 4096), (300, 1)]:
        lhs = O.rope(q, m, 10000.0) @ O.rope(k, n, 10000.0)
        rhs = O.rope(q, m - n, 10000.0) @ k
        assert abs(lhs - rhs) < 1e-9 * max(1.0, abs(lhs))


def test_rope_composition():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(32)
    np.testing.assert_allclose(O.rope(O.rope(x, 7, 500.0), 11, 500.0), O.rope(x, 18, 500.0), atol=1e-12)


def test_rope_pairs_are_half_split_and_angles_follow_base():
    # unit vector on component k must move only into component k + d/2 and
    # turn by pos * base^(-2k/d) (the RoFormer frequency ladder, NeoX pairing)
    d, base = 16, 10000.0
    for k in range(d // 2):
        e = np.zeros(d)
        e[k] = 1.0
        pos = 0.7
        y = O.rope(e, pos, base)
        others = [j for j in range(d) if j not in (k, k + d // 2)]
        assert np.all(y[others] == 0.0)
        ang = math.atan2(y[k + d // 2], y[k])
        assert abs(ang - pos * base ** (-2.0 * k / d)) < 1e-14


# ----------------------------------------------------------------------------
# attention + mask + GQA: against torch's scaled_dot_product_attention
# ----------------------------------------------------------------------------


def _tiny_forest_inputs(parent, prefix_lens, offs, Hq=4, Hkv=2, d=16, T=None, seed=0, pos=None):
    rng = np.random.default_rng(seed)
    n = len(parent)
    T = T if T is not None else int(max([o + l for o, l in zip(offs, prefix_lens)] + [1]))
    inp = {
        "parent": np.array(parent), "pos": np.array(pos if pos is not None else np.arange(n) + 50),
        "root_kv_off": np.array(offs), "root_kv_len": np.array(prefix_lens),
        "kv_k": rng.standard_normal((T, Hkv, d)).astype(np.float32),
        "kv_v": rng.standard_normal((T, Hkv, d)).astype(np.float32),
        "q_rows": rng.standard_normal((n, Hq, d)).astype(np.float32),
        "k_rows": rng.standard_normal((n, Hkv, d)).astype(np.float32),
        "v_rows": rng.standard_normal((n, Hkv, d)).astype(np.float32),
    }
    cfg = {"dtype": "f32", "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": d,
           "rope_base": 10000.0, "norm_eps": 1e-6}
    return cfg, inp


def _sdpa_reference(cfg, inp):
    """Attention of every row through torch SDPA (fp64) with a boolean mask
    built by walking the parent map in this test."""
    parent = [int(p) for p in inp["parent"]]
    n = len(parent)
    Hq, Hkv, d = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    # tree of each row and its root, found independently of the oracle
    root = []
    for i, p in enumerate(parent):
        root.append(i if p == -1 else root[p])
    roots = sorted(set(root))
    out = np.empty((n, Hq, d))
    kv_k = torch.tensor(inp["kv_k"], dtype=torch.float64)
    kv_v = torch.tensor(inp["kv_v"], dtype=torch.float64)
    for i in range(n):
        t = roots.index(root[i])
        off, ln = int(inp["root_kv_off"][t]), int(inp["root_kv_len"][t])
        anc = set()
        j = i
        while j != -1:
            anc.add(j)
            j = parent[j]
        rk = torch.tensor(np.stack([O.rope(inp["k_rows"][a].astype(np.float64), inp["pos"][a], 10000.0)
                                    for a in range(n)]))
        keys = torch.cat([kv_k[off:off + ln], rk], 0)                    # [ln + n, Hkv, d]
        vals = torch.cat([kv_v[off:off + ln], torch.tensor(inp["v_rows"], dtype=torch.float64)], 0)
        mask = torch.tensor([True] * ln + [a in anc for a in range(n)])
        q = torch.tensor(O.rope(inp["q_rows"][i].astype(np.float64), inp["pos"][i], 10000.0))
        G = Hq // Hkv
        K = keys.permute(1, 0, 2).repeat_interleave(G, 0)[None]          # [1, Hq, L, d]
        Vv = vals.permute(1, 0, 2).repeat_interleave(G, 0)[None]
        o = torch.nn.functional.scaled_dot_product_attention(q[None, :, None, :], K, Vv, attn_mask=mask[None, None, None, :])
        out[i] = o[0, :, 0, :].numpy()
    return out


def test_chain_attention_equals_causal_sdpa():
    parent = [-1, 0, 1, 2, 3, 4, 5, 6]
    cfg, inp = _tiny_forest_inputs(parent, [37], [0])
    att = O.attention_outputs(cfg, inp, range(8))
    ref = _sdpa_reference(cfg, inp)
    for i in range(8):
        np.testing.assert_allclose(att[i], ref[i], atol=1e-12)


def test_chain_attention_equals_is_causal_sdpa_on_packed_sequence():
    # the chain with an empty prefix is ordinary causal self-attention
    parent = [-1, 0, 1, 2, 3, 4]
    cfg, inp = _tiny_forest_inputs(parent, [0], [0], Hq=6, Hkv=3, d=8, T=1,
                                   pos=np.arange(6) + 9)
    att = O.attention_outputs(cfg, inp, range(6))
    q = torch.tensor(np.stack([O.rope(inp["q_rows"][i].astype(np.float64), 9 + i, 1e4) for i in range(6)]))
    k = torch.tensor(np.stack([O.rope(inp["k_rows"][i].astype(np.float64), 9 + i, 1e4) for i in range(6)]))
    v = torch.tensor(inp["v_rows"], dtype=torch.float64)
    o = torch.nn.functional.scaled_dot_product_attention(
        q.permute(1, 0, 2)[None], k.permute(1, 0, 2).repeat_interleave(2, 0)[None],
        v.permute(1, 0, 2).repeat_interleave(2, 0)[None], is_causal=True)[0].permute(1, 0, 2).numpy()
    for i in range(6):
        np.testing.assert_allclose(att[i], o[i], atol=1e-12)


def test_general_tree_attention_equals_masked_sdpa():
    # two trees, the first one branching; separate prefixes
    parent = [-1, 0, 0, 1, 2, 2, 5, -1, 7, 7, 8]
    cfg, inp = _tiny_forest_inputs(parent, [13, 6], [2, 20], T=30, Hq=6, Hkv=2, d=8)
    att = O.attention_outputs(cfg, inp, range(len(parent)))
    ref = _sdpa_reference(cfg, inp)
    for i in range(len(parent)):
        np.testing.assert_allclose(att[i], ref[i], atol=1e-12)


def test_single_visible_key_returns_its_value_and_equal_keys_average():
    # root with an empty prefix sees only itself: o = v_root for every head
    cfg, inp = _tiny_forest_inputs([-1], [0], [0], T=1)
    o = O.attention_outputs(cfg, inp, [0])[0]
    G = 2
    for h in range(4):
        np.testing.assert_array_equal(o[h], inp["v_rows"][0, h // G].astype(np.float64))
    # identical scores everywhere -> plain mean of the visible values
    keys = np.zeros((5, 1, 4))
    vals = np.arange(20, dtype=np.float64).reshape(5, 1, 4)
    o2 = O.attend(np.ones((3, 4)), keys, vals)
    np.testing.assert_allclose(o2, np.tile(vals[:, 0].mean(0), (3, 1)), atol=1e-14)


# ----------------------------------------------------------------------------
# projection + final norm + LM head: constructed weights
# ----------------------------------------------------------------------------


def test_project_norm_closed_forms():
    rng = np.random.default_rng(3)
    o = rng.standard_normal((4, 8))
    # identity W_o, eps = 0 -> unit RMS and scale invariance
    h = O.project_norm(np.eye(32), o, 0.0)
    assert abs(np.sqrt(np.mean(h * h)) - 1.0) < 1e-14
    np.testing.assert_allclose(O.project_norm(np.eye(32), 3.5 * o, 0.0), h, atol=1e-14)
    # constant vector c -> c / sqrt(c^2 + eps)
    c = 0.25
    h2 = O.project_norm(np.eye(32), np.full((4, 8), c), 1e-2)
    np.testing.assert_allclose(h2, c / np.sqrt(c * c + 1e-2), rtol=1e-15)
    # a permutation W_o permutes the (normalised) output; concat order is head-major
    perm = rng.permutation(32)
    P = np.eye(32)[perm]
    np.testing.assert_allclose(O.project_norm(P, o, 0.0), h[perm], atol=1e-14)
    assert O.project_norm(np.eye(32), np.zeros((4, 8)), 1e-6).tolist() == [0.0] * 32


def test_lm_head_indexing_with_one_hot_rows():
    hidden, V = 6, 20
    W = np.zeros((V, hidden), np.float32)
    for v in range(V):
        W[v, v % hidden] = v + 1
    h = np.arange(1, hidden + 1, dtype=np.float64)[None]
    cfg = {"dtype": "f32"}
    lg = O.lm_head(cfg, W, h, chunk=7)
    np.testing.assert_array_equal(lg[0], [(v + 1) * (v % hidden + 1) for v in range(V)])


def test_row_stats_ties_lse_gap():
    lg = np.array([1.0, 3.0, -2.0, 3.0, 0.5])
    m, lse, arg, gap = O.row_stats(lg)
    assert m == 3.0 and arg == 1 and gap == 0.0     # lowest index among ties
    from scipy.special import logsumexp
    assert abs(lse - logsumexp(lg)) < 1e-14
    c, V = -7.25, 4096
    m, lse, arg, gap = O.row_stats(np.full(V, c))
    assert abs(lse - (c + math.log(V))) < 1e-12 and arg == 0
    m, lse, arg, gap = O.row_stats(np.array([0.0, 2.0, 1.5]))
    assert arg == 1 and abs(gap - 0.5) < 1e-15


# ----------------------------------------------------------------------------
# overlap = 1 - TV
# ----------------------------------------------------------------------------


def test_overlap_is_one_minus_total_variation():
    rng = np.random.default_rng(4)
    for _ in range(20):
        p = O.softmax(rng.standard_normal(1000) * 2)
        q = O.softmax(rng.standard_normal(1000) * 2)
        ov = O.overlap(p, q)
        assert abs(ov - (1 - 0.5 * np.abs(p - q).sum())) < 1e-12
        assert abs(ov - O.overlap(q, p)) < 1e-15
        assert 0.0 <= ov <= 1.0
        assert abs(O.overlap(p, p) - 1.0) < 1e-12


def test_overlap_two_point_distributions_is_half():
    # p = (1/2, 1/2, 0, ...), q = (1/2, 0, 1/2, 0, ...) built from logits
    big = -2000.0
    lp = np.array([0.0, 0.0, big, big, big])
    lq = np.array([1.0, big, 1.0, big, big])
    assert O.overlap(O.softmax(lp), O.softmax(lq)) == 0.5
    # disjoint supports -> 0
    assert O.overlap(O.softmax(np.array([0.0, big])), O.softmax(np.array([big, 0.0]))) == 0.0


# ----------------------------------------------------------------------------
# acceptance
# ----------------------------------------------------------------------------


def test_acceptance_golden_examples():
    g = golden("acceptance_examples.json")
    for c in g["cases"]:
        n = len(c["greedy"])
        f = O.Forest([-1] + list(range(n - 1)))
        acc, bonus, last = O.accept_walk(f, 0, c["greedy"], c["drafts"])
        assert (acc, bonus, last) == (c["accept_len"], c["bonus"], c["last_row"]), c


def test_acceptance_on_branching_tree_takes_first_matching_child():
    #        0
    #      / | \
    #     1  2  3        greedy[0] = 4; drafts 1:4, 2:4, 3:9 -> child 1 (first)
    #     |     |
    #     4     5        greedy[1] = 6, drafts 4: 6 -> accepted
    parent = [-1, 0, 0, 0, 1, 3]
    f = O.Forest(parent)
    greedy = [4, 6, 0, 0, 8, 0]
    drafts = [0, 4, 4, 9, 6, 0]
    assert O.accept_walk(f, 0, greedy, drafts) == (3, 8, 4)
    drafts2 = [0, 3, 4, 4, 6, 0]            # row 2 is now the first match
    assert O.accept_walk(f, 0, greedy, drafts2) == (2, 0, 2)


def test_forest_rejects_bad_parent_maps():
    for bad in ([0], [-1, 1], [-1, 0, 3, 1], [-1, -1, 0], [1, -1]):
        with pytest.raises(ValueError):
            O.Forest(bad)


# ----------------------------------------------------------------------------
# survival
# ----------------------------------------------------------------------------


def test_survival_constant_alpha_closed_form():
    for alpha in (0.5, 0.3, 0.9):
        gamma = 7
        f = O.Forest([-1] + list(range(gamma)))
        s, sums = O.survival(f, [1.0] + [alpha] * gamma)
        for j in range(gamma + 1):
            assert abs(s[j] - alpha ** j) < 1e-15
        assert abs(sums[0] - ((1 - alpha ** (gamma + 1)) / (1 - alpha) - 1)) < 1e-14


def test_survival_compounding_golden():
    g = golden("compounding_gamma7.json")
    gamma, eps = g["gamma"], g["per_position_overestimate"]
    f = O.Forest([-1] + list(range(gamma)))
    rng = np.random.default_rng(5)
    alpha = rng.uniform(0.3, 0.8, gamma)
    s_true, _ = O.survival(f, [1.0] + list(alpha))
    s_over, _ = O.survival(f, [1.0] + list(alpha * (1 + eps)))
    over = s_over[gamma] / s_true[gamma] - 1
    assert abs(over - g["final_overestimate_approx"]) <= g["abs_tolerance"]


def test_expected_tokens_tend_to_speedup_bound():
    g = golden("speedup_bound.json")
    for c in g["cases"]:
        gamma = 400
        f = O.Forest([-1] + list(range(gamma)))
        _, sums = O.survival(f, [1.0] + [c["alpha"]] * gamma)
        assert abs((1 + sums[0]) - c["limit"]) < 1e-9


def test_survival_on_tree_multiplies_along_paths():
    parent = [-1, 0, 0, 1, 1, 3]
    ov = [1.0, 0.5, 0.25, 0.5, 0.125, 0.5]
    s, sums = O.survival(O.Forest(parent), ov)
    assert s.tolist() == [1.0, 0.5, 0.25, 0.25, 0.0625, 0.125]
    assert sums[0] == 0.5 + 0.25 + 0.25 + 0.0625 + 0.125


# ----------------------------------------------------------------------------
# byte accounting used for roofline figures
# ----------------------------------------------------------------------------


def test_kv_bytes_per_token_golden():
    from draft_block_verification_verify_amd.accounting import kv_bytes_per_token
    g = golden("kv_bytes_per_token.json")
    t, dft = g["target"], g["drafter"]
    bt = kv_bytes_per_token(t["layers"], t["kv_heads"], t["head_dim"], t["bytes_per_el"])
    assert bt == t["bytes_per_token"]
    assert bt * t["context"] / 2 ** 30 == t["total_gib"]
    bd = kv_bytes_per_token(dft["layers"], dft["kv_heads"], dft["head_dim"], dft["bytes_per_el"])
    assert bd == dft["bytes_per_token"]
    assert bd * dft["window"] / 2 ** 20 == dft["per_request_mib"]
    assert bd * dft["window"] * dft["concurrent"] / 2 ** 30 == dft["total_gib"]
