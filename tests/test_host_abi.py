"""CPU tests of the boundary: the built library loads and exports every
symbol include/spec_verify.h declares, create() rejects bad configurations
before touching a device, and the host planner (validation, ancestor masks,
attention work list) behaves, via a g++ build of plan.cpp."""
import ctypes as C
import os
import re
import subprocess

import numpy as np
import pytest

from draft_block_verification_verify_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")
CSRC = os.path.join(ROOT, "draft_block_verification_verify_amd", "csrc")


@pytest.fixture(scope="session")
def libsv():
    if not os.path.exists(B.LIB_PATH):
        from draft_block_verification_verify_amd import build
        build.build()
    return B.lib()


def declared_functions():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"\b(spec_verify_\w+)\s*\(", txt)))


def test_library_exports_every_declared_symbol(libsv):
    names = declared_functions()
    assert set(names) == set(B.SYMBOLS), names
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (\w+)", out))
    for n in names:
        assert n in exported, n
        assert getattr(libsv, n) is not None


def good_cfg(**kw):
    c = dict(n_q_heads=4, n_kv_heads=2, head_dim=64, hidden=256, vocab=4096, dtype=B.SV_F32,
             rope_base=10000.0, norm_eps=1e-6, max_rows=8, max_roots=1, max_tree_rows=8, max_pos=200)
    c.update(kw)
    return B.SvConfig(**c)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), B.SV_ERR_UNSUPPORTED),
    (dict(n_q_heads=5), B.SV_ERR_INVALID_ARG),
    (dict(hidden=100), B.SV_ERR_UNSUPPORTED),
    (dict(vocab=1), B.SV_ERR_INVALID_ARG),
    (dict(dtype=7), B.SV_ERR_INVALID_ARG),
    (dict(max_tree_rows=65), B.SV_ERR_INVALID_ARG),
    (dict(max_rows=0), B.SV_ERR_INVALID_ARG),
    (dict(rope_base=0.5), B.SV_ERR_INVALID_ARG),
    (dict(norm_eps=-1.0), B.SV_ERR_INVALID_ARG),
])
def test_create_rejects_bad_config_before_device(libsv, kw, status):
    h = C.c_void_p()
    st = libsv.spec_verify_create(C.byref(good_cfg(**kw)), C.c_void_p(16), C.c_void_p(16), C.byref(h))
    assert st == status, B.spec_verify_last_error()
    assert h.value is None
    assert B.spec_verify_last_error() != ""


def test_create_null_weights_and_null_handle_calls(libsv):
    h = C.c_void_p()
    assert libsv.spec_verify_create(C.byref(good_cfg()), None, C.c_void_p(16), C.byref(h)) == B.SV_ERR_INVALID_ARG
    assert libsv.spec_verify_run(None, None, None, None) == B.SV_ERR_INVALID_ARG
    assert libsv.spec_verify_destroy(None) == B.SV_OK
    assert libsv.spec_verify_profile(None, 1) == B.SV_ERR_INVALID_ARG


def test_create_without_gpu_fails_loudly(libsv):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    h = C.c_void_p()
    st = libsv.spec_verify_create(C.byref(good_cfg()), C.c_void_p(16), C.c_void_p(16), C.byref(h))
    assert st in (B.SV_ERR_HIP, B.SV_ERR_UNSUPPORTED)
    assert h.value is None


# ----------------------------------------------------------------------------
# host planner (g++ build, no HIP)
# ----------------------------------------------------------------------------


@pytest.fixture(scope="session")
def plan_lib(tmp_path_factory):
    d = tmp_path_factory.mktemp("svplan")
    so = str(d / "libsvplan.so")
    cmd = ["g++", "-O1", "-std=c++17", "-shared", "-fPIC", "-I", CSRC,
           os.path.join(CSRC, "plan.cpp"), os.path.join(ROOT, "tests", "native", "plan_capi.cpp"), "-o", so]
    subprocess.run(cmd, check=True)
    L = C.CDLL(so)
    L.svp_plan.restype = C.c_int
    return L


def plan(L, dims, parent, pos, off, lens, kv_tokens, slot_cap=1 << 20, target=1024):
    parent = np.ascontiguousarray(parent, np.int32)
    pos = np.ascontiguousarray(pos, np.int32)
    off = np.ascontiguousarray(off, np.int64)
    lens = np.ascontiguousarray(lens, np.int32)
    n = len(parent)
    dims = np.ascontiguousarray(dims, np.int32)
    stats = np.zeros(9, np.int64)
    err = C.create_string_buffer(512)
    anc = np.zeros(max(n, 1), np.uint64)
    items = np.zeros((8192, 14), np.int32)       # AttnItem: 10 int32, one int64, kv_min, pad
    runs = np.zeros((8192, 4), np.int32)         # AttnRun: first, count, tiles, pad
    st = L.svp_plan(dims.ctypes.data_as(C.c_void_p), n, len(lens), parent.ctypes.data_as(C.c_void_p),
                    pos.ctypes.data_as(C.c_void_p), off.ctypes.data_as(C.c_void_p),
                    lens.ctypes.data_as(C.c_void_p), C.c_int64(kv_tokens), C.c_int64(slot_cap), target,
                    stats.ctypes.data_as(C.c_void_p), err, 512, anc.ctypes.data_as(C.c_void_p),
                    items.ctypes.data_as(C.c_void_p), 8192, runs.ctypes.data_as(C.c_void_p), 8192)
    if st != 0:
        return st, err.value.decode(), stats, anc, None
    check_runs(items[: stats[2]], runs[: stats[8]], stats, 8192 // dims[2], target)
    return st, err.value.decode(), stats, anc, items[: stats[2]]


def check_runs(items, runs, stats, KT, target):
    """Runs cut the item sequence in order: run j holds items
    [first, first + count), its tiles sum to `tiles`, every run but the last
    has chunk / KT tiles, and no more runs than asked for."""
    assert 1 <= len(runs) <= target
    ch = stats[4] // KT
    nxt = 0
    for j, (first, count, tiles, _) in enumerate(runs):
        assert first == nxt and count >= 1
        nxt = first + count
        its = items[first:first + count]
        assert tiles == sum((it[5] - it[4]) // KT for it in its)
        assert tiles == ch or (j == len(runs) - 1 and 1 <= tiles <= ch)
        # only a run's first item may start inside a group, only its last end inside one
        for it in its[1:]:
            assert it[4] == 0
    assert nxt == len(items)


DIMS = [32, 8, 128, 4096, 151936, 1, 512, 64, 64, 1 << 20]   # Hq Hkv d hidden V dtype rows roots tree pos


def test_plan_ancestor_masks_and_items_cover_keys(plan_lib):
    parent = [-1, 0, 0, 1, 2, 2, 5, -1, 7, 8]
    lens, off = [300, 0], [5, 0]
    st, err, stats, anc, items = plan(plan_lib, DIMS, parent, np.arange(10) + 400, off, lens, 305)
    assert st == 0, err
    # ancestor-or-self masks by brute force
    starts = [0, 7]
    for i, p in enumerate(parent):
        s = max(x for x in starts if x <= i)
        bits, j = 0, i
        while j != -1:
            bits |= 1 << (j - s)
            j = parent[j]
        assert int(anc[i]) == bits, i
    # items: per (tree, kv head, query group) the tile-aligned key ranges cover
    # the tree's key sequence: ceil(len / KT) prefix tiles, then ceil(T / KT)
    # row tiles (KT = 8192 / d = 64 keys)
    T = [7, 3]
    G = 4
    KT = 8192 // DIMS[2]
    assert stats[0] == 2 and stats[1] == 8
    slots = []
    for tree in range(2):
        for g in range(8):
            for qg in range((T[tree] * G + 127) // 128):
                its = [it for it in items if it[0] == tree and it[1] == g and it[2] == qg * 128]
                its.sort(key=lambda it: it[4])
                span = (-(-lens[tree] // KT) - (-T[tree] // KT)) * KT
                assert its[0][4] == 0 and its[-1][5] == span
                for a, b in zip(its, its[1:]):
                    assert a[5] == b[4]
                assert all(it[4] % KT == 0 and it[5] % KT == 0 and it[5] > it[4] for it in its)
                for it in its:
                    assert it[3] == min(128, T[tree] * G - qg * 128)
                    slots.append((it[6], it[6] + it[3]))
                    # the tree's own fields, copied into every item
                    assert (it[7], it[8], it[9]) == (starts[tree], T[tree], lens[tree])
                    assert int(it[10:12].view(np.int64)[0]) == off[tree]
    slots.sort()
    assert slots[0][0] == 0 and slots[-1][1] == stats[3]
    for a, b in zip(slots, slots[1:]):
        assert a[1] == b[0]
    assert stats[6] <= stats[7]          # fits the handle's metadata capacity


def test_plan_coarsens_split_to_fit_slot_capacity(plan_lib):
    parent = [-1] + list(range(16))
    st, err, stats, _, items = plan(plan_lib, [24, 4, 256, 5120, 248320, 1, 17, 1, 64, 1 << 20],
                                    parent, np.arange(17) + 8192, [0], [8192], 8192, slot_cap=24 * 17 * 2)
    assert st == 0, err
    assert stats[3] <= 24 * 17 * 2
    # 4 KV heads x 257 tiles in runs of at least 208 tiles: at most 2 items per head
    assert stats[4] // 32 >= 208 and len(items) <= 8
    for g in range(4):
        assert 1 <= sum(1 for it in items if it[1] == g) <= 2


def test_plan_runs_fit_resident_workgroups(plan_lib):
    # one 17-row chain at 27B shape: 102 query vectors per group take the
    # eight-wave attention launch (one workgroup per compute unit), so the
    # 4 x 257 tiles are cut into at most target / 2 runs (one round); 8-row
    # chains (32 query vectors, four-wave launch) may use up to target runs
    parent = [-1] + list(range(16))
    dims = [24, 4, 256, 5120, 248320, 1, 17, 1, 64, 1 << 20]
    st, err, stats, _, items = plan(plan_lib, dims, parent, np.arange(17) + 8192, [0], [8192], 8192, target=512)
    assert st == 0, err
    assert stats[8] <= 256
    KT = 32
    assert stats[8] == -(-(4 * 257) // (stats[4] // KT))
    parent8 = [-1] + list(range(7))
    dims8 = [32, 8, 128, 4096, 151936, 1, 8, 1, 64, 1 << 20]
    st, err, stats8, _, _ = plan(plan_lib, dims8, parent8, np.arange(8) + 4096, [0], [4096], 4096, target=512)
    assert st == 0, err
    assert 256 < stats8[8] <= 512


def test_plan_packs_trees_over_one_kv_segment(plan_lib):
    # Trees that read the same KV segment (same offset) share one query group
    # per KV head: up to 64 rows and 128 query vectors, prefix lengths within
    # a factor 2.  Here: three 7-row chains on segment 0 (lengths 100, 120,
    # 150: one pack), a fourth on segment 0 with length 400 (too long: its
    # own pack), a fifth on another segment (its own pack).
    T = 7
    lens = [100, 120, 150, 400, 90]
    offs = [0, 0, 0, 0, 1000]
    parent = []
    for t in range(5):
        parent += [-1] + [t * T + j for j in range(T - 1)]
    n = len(parent)
    pos = np.concatenate([np.arange(T) + lens[t] for t in range(5)])
    st, err, stats, anc, items = plan(plan_lib, DIMS, parent, pos, offs, lens, 1200)
    assert st == 0, err
    L = plan_lib
    L.svp_packs.restype = C.c_int
    rp, rl, rk = (np.zeros(n, np.int32) for _ in range(3))
    ra = np.zeros(n, np.uint64)
    args = [np.ascontiguousarray(x) for x in (np.array(DIMS, np.int32), np.array(parent, np.int32),
                                              pos.astype(np.int32), np.array(offs, np.int64),
                                              np.array(lens, np.int32))]
    npk = L.svp_packs(args[0].ctypes.data_as(C.c_void_p), n, 5, args[1].ctypes.data_as(C.c_void_p),
                      args[2].ctypes.data_as(C.c_void_p), args[3].ctypes.data_as(C.c_void_p),
                      args[4].ctypes.data_as(C.c_void_p), C.c_int64(1200), rp.ctypes.data_as(C.c_void_p),
                      rl.ctypes.data_as(C.c_void_p), rk.ctypes.data_as(C.c_void_p), ra.ctypes.data_as(C.c_void_p))
    assert npk == 3
    assert rp.tolist() == [0] * 21 + [1] * 7 + [2] * 7
    starts = [0, 0, 0, 21, 28]
    assert rl.tolist() == [i - starts[i // T] for i in range(n)]
    assert rk.tolist() == sum(([lens[t]] * T for t in range(5)), [])
    for i in range(n):
        t = i // T
        shift = t * T - starts[t]
        assert int(ra[i]) == int(anc[i]) << shift, i
    # items are per pack: the pack's first row, its rows and longest prefix,
    # and its key range covers that prefix and the pack's rows
    KT = 8192 // DIMS[2]
    for pk, (start, rows, klen, off) in enumerate([(0, 21, 150, 0), (21, 7, 400, 0), (28, 7, 90, 1000)]):
        its = [it for it in items if it[0] == pk]
        assert its and all((it[7], it[8], it[9]) == (start, rows, klen) for it in its)
        assert all(int(it[10:12].view(np.int64)[0]) == off for it in its)
        for g in range(DIMS[1]):
            gi = sorted((it for it in its if it[1] == g), key=lambda it: it[4])
            assert gi[0][4] == 0 and gi[-1][5] == (-(-klen // KT) - (-rows // KT)) * KT
            assert all(it[3] == rows * 4 for it in gi)


def test_plan_caps_splits_per_group(plan_lib):
    # one long prefix and a huge work-item target: the split count per
    # (tree, KV head, query group) stays within what the merge handles
    st, err, stats, _, items = plan(plan_lib, DIMS, [-1, 0], [500000, 500001], [0], [500000], 500000,
                                    target=100000)
    assert st == 0, err
    per_head = {}
    for it in items:
        per_head[it[1]] = per_head.get(it[1], 0) + 1
    assert max(per_head.values()) <= 1024


@pytest.mark.parametrize("parent,pos,off,lens,kv,code,frag", [
    ([0, 0], [1, 2], [0], [1], 4, -2, "root"),
    ([-1, 2, 1], [1, 2, 3], [0], [1], 4, -2, "parent"),
    ([-1, 0, -1, 0], [1, 2, 3, 4], [0, 0], [1, 1], 4, -2, "parent"),
    ([-1, 0], [1, 2], [0, 0], [1, 1], 4, -2, "roots"),
    ([-1, 0], [1, 1 << 20], [0], [1], 4, -2, "position"),
    ([-1, 0], [1, -1], [0], [1], 4, -2, "position"),
    ([-1, 0], [1, 2], [3], [2], 4, -2, "prefix"),
    ([-1, 0], [1, 2], [0], [-1], 4, -2, "prefix"),
])
def test_plan_rejects_bad_trees(plan_lib, parent, pos, off, lens, kv, code, frag):
    st, err, *_ = plan(plan_lib, DIMS, parent, pos, off, lens, kv)
    assert st == code and frag in err, (st, err)


def test_plan_capacities(plan_lib):
    dims = list(DIMS)
    dims[6], dims[7] = 4, 1          # max_rows, max_roots
    st, err, *_ = plan(plan_lib, dims, [-1, 0, 1, 2, 3], range(5), [0], [1], 1)
    assert st == B.SV_ERR_CAPACITY and "max_rows" in err
    dims = list(DIMS)
    dims[8] = 4          # max_tree_rows
    st, err, *_ = plan(plan_lib, dims, [-1, 0, 1, 2, 3], range(5), [0], [1], 1)
    assert st == B.SV_ERR_CAPACITY and "max_tree_rows" in err
    dims = list(DIMS)
    dims[7] = 1          # max_roots
    st, err, *_ = plan(plan_lib, dims, [-1, -1], range(2), [0, 0], [1, 1], 1)
    assert st == B.SV_ERR_CAPACITY and "max_roots" in err


def test_run_static_rejects_before_device(libsv):
    # the allocation-free entry point: configuration, dtype and argument
    # errors come back before any device call (no GPU needed here)
    inp = B.SvInputs()
    out = B.SvOutputs()
    f = libsv.spec_verify_run_static
    assert f(None, C.c_void_p(16), C.c_void_p(16), C.byref(inp), C.byref(out), None) == B.SV_ERR_INVALID_ARG
    assert f(C.byref(good_cfg()), None, C.c_void_p(16), C.byref(inp), C.byref(out), None) == B.SV_ERR_INVALID_ARG
    assert f(C.byref(good_cfg(dtype=B.SV_BF16)), C.c_void_p(16), C.c_void_p(16), C.byref(inp), C.byref(out),
             None) == B.SV_ERR_UNSUPPORTED
    assert "fp32" in B.spec_verify_last_error()
    assert f(C.byref(good_cfg(head_dim=96)), C.c_void_p(16), C.c_void_p(16), C.byref(inp), C.byref(out),
             None) == B.SV_ERR_UNSUPPORTED
    # a valid tree whose rows are not given: refused by the argument checks
    parent = np.array([-1, 0], np.int32)
    pos = np.array([3, 4], np.int32)
    off = np.array([0], np.int64)
    ln = np.array([3], np.int32)
    inp = B.SvInputs(2, 1, parent.ctypes.data_as(C.POINTER(C.c_int32)), pos.ctypes.data_as(C.POINTER(C.c_int32)),
                     off.ctypes.data_as(C.POINTER(C.c_int64)), ln.ctypes.data_as(C.POINTER(C.c_int32)), 3,
                     16, 16, 0, 0, 0, 0, 0, 0, 0, 0)
    assert f(C.byref(good_cfg()), C.c_void_p(16), C.c_void_p(16), C.byref(inp), C.byref(out),
             None) == B.SV_ERR_INVALID_ARG
    # misaligned weights
    assert f(C.byref(good_cfg()), C.c_void_p(20), C.c_void_p(16), C.byref(inp), C.byref(out),
             None) == B.SV_ERR_INVALID_ARG


def test_prepared_weight_bytes_and_refusals(libsv):
    # host-only: the prepared-weights buffer's size is fixed by hidden,
    # n_q_heads * head_dim and vocab (three 256-byte aligned parts and a
    # 256-byte check word), not by the capacities; other dtypes and the FP8
    # format are refused, and every call checks its arguments before any
    # device work
    def al(x):
        return (x + 255) // 256 * 256

    def blocked(rows, k):
        return (rows + 255) // 256 * 256 * k

    cfg = good_cfg(dtype=B.SV_BF16)
    h, k, v = cfg.hidden, cfg.n_q_heads * cfg.head_dim, cfg.vocab
    want = al(h * k * 2) + al(blocked(h, k) * 2) + al(blocked(v, h) * 2) + 256
    assert B.spec_verify_weight_bytes(cfg) == want
    assert B.spec_verify_weight_bytes(good_cfg(dtype=B.SV_BF16, max_rows=7, max_roots=1)) == want
    n = C.c_size_t(7)
    assert libsv.spec_verify_weight_bytes(C.byref(good_cfg()), C.byref(n)) == B.SV_ERR_UNSUPPORTED and n.value == 0
    assert libsv.spec_verify_weight_bytes(C.byref(good_cfg(dtype=B.SV_BF16, weight_format=B.SV_WEIGHTS_FP8)),
                                          C.byref(n)) == B.SV_ERR_UNSUPPORTED
    assert libsv.spec_verify_weight_bytes(None, C.byref(n)) == B.SV_ERR_INVALID_ARG
    assert libsv.spec_verify_weight_bytes(C.byref(cfg), None) == B.SV_ERR_INVALID_ARG
    prep = libsv.spec_verify_prepare_weights
    assert prep(C.byref(cfg), None, C.c_void_p(256), C.c_void_p(256), None) == B.SV_ERR_INVALID_ARG
    assert prep(C.byref(cfg), C.c_void_p(256), C.c_void_p(256), C.c_void_p(272), None) == B.SV_ERR_INVALID_ARG
    assert prep(C.byref(good_cfg()), C.c_void_p(256), C.c_void_p(256), C.c_void_p(256), None) == B.SV_ERR_UNSUPPORTED
    hp = C.c_void_p(1)
    create = libsv.spec_verify_create_prepared
    assert create(C.byref(cfg), None, C.byref(hp)) == B.SV_ERR_INVALID_ARG and hp.value is None
    assert create(C.byref(cfg), C.c_void_p(272), C.byref(hp)) == B.SV_ERR_INVALID_ARG
    assert create(C.byref(good_cfg()), C.c_void_p(256), C.byref(hp)) == B.SV_ERR_UNSUPPORTED
