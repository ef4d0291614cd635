"""CPU tests of host and shared native code, built with g++ (no GPU, no HIP):

* the e4m3 encoder and scale exponent of the FP8 LM head (k_fp8.hpp, the same
  source the device compiles) against the oracle's e4m3 rounding and
  power-of-two scales, over every bf16 value and every scale boundary;
* the alignment check spec_verify_run makes before it enqueues anything;
* the planner (plan.cpp) and the verify-budget schedule (schedule.cpp) under
  AddressSanitizer and UndefinedBehaviorSanitizer, on valid and invalid
  trees, layouts and schedules, with the same results as the plain build.
"""
import ctypes as C
import os
import subprocess

import numpy as np
import pytest

from draft_block_verification_verify_amd import binding as B
from oracle import verify_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "draft_block_verification_verify_amd", "csrc")
NATIVE = os.path.join(ROOT, "tests", "native")


@pytest.fixture(scope="module")
def fp8lib(tmp_path_factory):
    so = str(tmp_path_factory.mktemp("svfp8") / "libsvfp8.so")
    subprocess.run(["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-I", CSRC,
                    os.path.join(NATIVE, "fp8_capi.cpp"), "-o", so], check=True)
    L = C.CDLL(so)
    L.svp_fp8_weight_ok.restype = C.c_int
    L.svp_fp8_weight_ok.argtypes = [C.c_float]
    return L


def _codes(L, x, e):
    x = np.ascontiguousarray(x, np.float32)
    e = np.ascontiguousarray(np.broadcast_to(e, x.shape), np.int32)
    out = np.zeros(x.shape, np.uint32)
    L.svp_e4m3_codes(x.ctypes.data_as(C.c_void_p), e.ctypes.data_as(C.c_void_p), out.ctypes.data_as(C.c_void_p),
                     C.c_int64(x.size))
    return out


def _values(L, codes):
    codes = np.ascontiguousarray(codes, np.uint32)
    out = np.zeros(codes.shape, np.float32)
    L.svp_e4m3_values(codes.ctypes.data_as(C.c_void_p), out.ctypes.data_as(C.c_void_p), C.c_int64(codes.size))
    return out.astype(np.float64)


def _exponents(L, amax):
    amax = np.ascontiguousarray(amax, np.float32)
    out = np.zeros(amax.shape, np.int32)
    L.svp_fp8_exponents(amax.ctypes.data_as(C.c_void_p), out.ctypes.data_as(C.c_void_p), C.c_int64(amax.size))
    return out


def _all_bf16(finite_only=True):
    bits = np.arange(1 << 16, dtype=np.uint32)
    v = (bits << 16).view(np.float32)
    return v[np.isfinite(v)] if finite_only else v


def test_scale_exponent_matches_the_oracle_for_every_bf16_value(fp8lib):
    v = _all_bf16()
    a = np.abs(v)
    e = _exponents(fp8lib, a)
    want = O.pow2_scales(a.astype(np.float64))
    np.testing.assert_array_equal(np.exp2(e.astype(np.float64)), want)


@pytest.mark.parametrize("k", [-126, -20, -9, -8, 0, 7, 100, 119])
def test_scale_exponent_at_boundaries(fp8lib, k):
    # 448 * 2^k sits exactly on a boundary: its exponent is k; one fp32 ulp
    # above it takes k + 1 (unless the floor -126 holds)
    b = np.float32(448.0) * np.float32(2.0) ** np.float32(k) if k > -127 else None
    amax = np.array([b, np.nextafter(b, np.float32(np.inf)), np.nextafter(b, np.float32(0))], np.float32)
    e = _exponents(fp8lib, amax)
    assert e[0] == max(k, -126) and e[1] == max(k + 1, -126) and e[2] == max(k, -126)
    np.testing.assert_array_equal(np.exp2(e.astype(np.float64)), O.pow2_scales(amax.astype(np.float64)))


def test_scale_exponent_special_values(fp8lib):
    amax = np.array([0.0, np.inf, np.nan, 1e-45, 1e-38, 3.4e38], np.float32)
    e = _exponents(fp8lib, amax)
    assert e[0] == 0 and e[1] == 0 and e[2] == 0           # no scale for nothing or a value that is not finite
    assert e[3] == -126 and e[4] == -126                     # the floor: scales stay normal fp32 numbers
    assert e[5] == 120 and 3.4e38 <= 448.0 * 2.0 ** 120
    assert fp8lib.svp_fp8_weight_ok(1.0) == 1 and fp8lib.svp_fp8_weight_ok(-3.3e38) == 1
    assert fp8lib.svp_fp8_weight_ok(float("inf")) == 0 and fp8lib.svp_fp8_weight_ok(float("nan")) == 0


def test_weight_codes_equal_the_oracles(fp8lib):
    # a weight w with row exponent e is stored as the code of w / 2^e: every
    # finite bf16 value at every exponent that keeps |w / 2^e| <= 448
    v = _all_bf16().astype(np.float32)
    a = np.abs(v.astype(np.float64))
    nz = a > 0
    e_min = _exponents(fp8lib, np.abs(v))               # the smallest valid exponent of a row holding v alone
    for de in (0, 1, 3):
        e = (e_min + de).astype(np.int32)
        codes = _codes(fp8lib, v, e)
        got = _values(fp8lib, codes)
        want = O.e4m3(v.astype(np.float64) / np.exp2(e.astype(np.float64)))
        np.testing.assert_array_equal(got[nz], want[nz])
        assert (got[~nz] == 0).all()
        # the sign bit follows the value's sign (zero keeps its sign bit)
        assert ((codes >> 7) & 1 == (v < 0) | ((v == 0) & np.signbit(v))).all()


def test_encoder_midpoints_round_half_to_even(fp8lib):
    vals = np.unique(np.abs(O.e4m3(np.linspace(0, 448, 200001))))
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([mids, np.nextafter(mids.astype(np.float32), np.float32(0)).astype(np.float64),
                        np.nextafter(mids.astype(np.float32), np.float32(np.inf)).astype(np.float64)])
    x = np.concatenate([x, -x]).astype(np.float32)
    got = _values(fp8lib, _codes(fp8lib, x, 0))
    np.testing.assert_array_equal(got, O.e4m3(x.astype(np.float64)))


def test_encoder_out_of_range_inputs_saturate_or_give_nan(fp8lib):
    codes = _codes(fp8lib, np.array([449.0, -1e30, np.inf, np.nan], np.float32), 0)
    assert codes.tolist()[:3] == [0x7E, 0xFE, 0x7E] and (codes[3] & 0x7F) == 0x7F


# ----------------------------------------------------------------------------
# alignment of a run's device buffers
# ----------------------------------------------------------------------------


@pytest.fixture(scope="module")
def planlib(tmp_path_factory):
    so = str(tmp_path_factory.mktemp("svplan2") / "libsvplan.so")
    subprocess.run(["g++", "-O1", "-std=c++17", "-shared", "-fPIC", "-I", CSRC, os.path.join(CSRC, "plan.cpp"),
                    os.path.join(NATIVE, "plan_capi.cpp"), "-o", so], check=True)
    L = C.CDLL(so)
    L.svp_check_alignment.restype = C.c_int
    return L


WIDE = ["kv_k", "kv_v", "q_rows", "k_rows", "v_rows", "drafter_logits", "logits"]
NARROW = ["draft_ids", "u_accept", "u_bonus", "accept_len", "bonus", "last_row", "surv_sum", "argmax", "row_max",
          "row_lse", "overlap", "survival"]


def _align(L, wide, narrow):
    w = (C.c_void_p * 7)(*wide)
    n = (C.c_void_p * 12)(*narrow)
    err = C.create_string_buffer(256)
    return L.svp_check_alignment(w, n, err, 256), err.value.decode()


def test_alignment_check_names_the_offending_buffer(planlib):
    base = 1 << 20
    ok_w, ok_n = [base + 64 * i for i in range(7)], [base + 4096 + 16 * i for i in range(12)]
    assert _align(planlib, ok_w, ok_n) == (0, "")
    for i, name in enumerate(WIDE):
        for off in (4, 8, 12):
            w = list(ok_w)
            w[i] += off
            st, err = _align(planlib, w, ok_n)
            assert st == B.SV_ERR_INVALID_ARG and name in err and "16-byte" in err
    for i, name in enumerate(NARROW):
        n = list(ok_n)
        n[i] += 2
        st, err = _align(planlib, ok_w, n)
        assert st == B.SV_ERR_INVALID_ARG and name in err and "4-byte" in err
        n[i] += 2                        # 4-byte aligned is enough for these
        assert _align(planlib, ok_w, n)[0] == 0
    # null pointers (optional buffers) pass this check
    assert _align(planlib, [None] * 7, [None] * 12)[0] == 0


# ----------------------------------------------------------------------------
# planner and schedule under ASan + UBSan
# ----------------------------------------------------------------------------


def _plan_cases():
    r = np.random.default_rng(21)
    dims = [32, 8, 128, 4096, 151936, 1, 512, 64, 64, 1 << 20]
    cases = []

    def add(d, parent, pos, off, lens, kv, slot_cap=1 << 20, target=1024):
        cases.append((list(d), list(parent), list(pos), list(off), list(lens), kv, slot_cap, target))

    # the planner tests' trees
    add(dims, [-1, 0, 0, 1, 2, 2, 5, -1, 7, 8], np.arange(10) + 400, [5, 0], [300, 0], 305)
    add([24, 4, 256, 5120, 248320, 1, 17, 1, 64, 1 << 20], [-1] + list(range(16)), np.arange(17) + 8192, [0], [8192],
        8192, 24 * 17 * 2)
    add([24, 4, 256, 5120, 248320, 1, 17, 1, 64, 1 << 20], [-1] + list(range(16)), np.arange(17) + 8192, [0], [8192],
        8192, 1 << 20, 512)
    add(dims, [-1, 0], [500000, 500001], [0], [500000], 500000, 1 << 20, 100000)
    # shared segments (packs), lone roots, empty prefixes, a 64-row chain
    T, lens, offs = 7, [100, 120, 150, 400, 90], [0, 0, 0, 0, 1000]
    par = []
    for t in range(5):
        par += [-1] + [t * T + j for j in range(T - 1)]
    add(dims, par, np.concatenate([np.arange(T) + L for L in lens]), offs, lens, 1200)
    add(dims, [-1] + list(range(63)) + [-1, -1], list(range(66)), [0, 10, 10], [5, 0, 3], 20)
    # random forests over random segments, several head shapes
    for d, hq, hkv in [(64, 4, 2), (128, 32, 8), (256, 24, 4)]:
        for _ in range(12):
            R = int(r.integers(1, 12))
            par, pos, off, lens = [], [], [], []
            tok = int(r.integers(0, 3000))
            for _t in range(R):
                nt = int(r.integers(1, 20))
                s = len(par)
                par += [-1] + [s + int(r.integers(0, j)) for j in range(1, nt)]
                L = int(r.integers(0, 600))
                o = int(r.integers(0, max(1, tok - L))) if r.random() < 0.5 else 0
                off.append(o)
                lens.append(min(L, tok - o) if tok > o else 0)
                pos += list(range(lens[-1], lens[-1] + nt))
            add([hq, hkv, d, 1024, 5000, 1, 256, 16, 64, 1 << 20], par, pos, off, lens, tok,
                int(r.integers(2000, 1 << 20)), int(r.integers(1, 600)))
    # invalid inputs: every rejection path
    for par, pos, off, lens, kv in [([0, 0], [1, 2], [0], [1], 4), ([-1, 2, 1], [1, 2, 3], [0], [1], 4),
                                    ([-1, 0], [1, 1 << 20], [0], [1], 4), ([-1, 0], [1, -1], [0], [1], 4),
                                    ([-1, 0], [1, 2], [3], [2], 4), ([-1, 0], [1, 2], [0], [-1], 4),
                                    ([-1, 0, 1, 2, 3], range(5), [0], [1], 1)]:
        add(dims, par, pos, off, lens, kv)
    small = list(dims)
    small[6], small[7] = 4, 1
    add(small, [-1, 0, 1, 2, 3], range(5), [0], [1], 1)
    add([5, 2, 128, 64, 100, 1, 8, 1, 8, 100], [-1], [0], [0], [0], 0)         # bad head counts
    add([4, 2, 96, 64, 100, 1, 8, 1, 8, 100], [-1], [0], [0], [0], 0)          # bad head dim
    return cases


def _schedule_cases():
    r = np.random.default_rng(5)
    cases = []
    for _ in range(120):
        nr = int(r.integers(1, 6))
        n_cand = [int(r.integers(0, 7)) for _ in range(nr)]
        par, conf = [], []
        for k in n_cand:
            par += [int(r.integers(-1, j)) if r.random() < 0.5 else j - 1 for j in range(k)]
            conf += r.uniform(0, 1, k).round(4).tolist()
        npts = int(r.integers(1, 5))
        rows = np.sort(r.choice(np.arange(1, 40), npts, replace=False)).tolist()
        ms = np.cumsum(r.uniform(0.05, 1, npts)).round(4).tolist()
        cases.append((n_cand, par, conf, rows, ms, int(r.integers(0, 12)) if r.random() < 0.3 else 0))
    # invalid: a bad parent, a confidence outside [0, 1], a decreasing curve, a cap below the request count
    cases.append(([2], [-1, 1], [0.5, 0.5], [1, 2], [1.0, 2.0], 0))
    cases.append(([1], [-1], [1.5], [1, 2], [1.0, 2.0], 0))
    cases.append(([1], [-1], [0.5], [2, 1], [1.0, 2.0], 0))
    cases.append(([1, 1], [-1, -1], [0.5, 0.5], [1, 2], [1.0, 2.0], 1))
    return cases


def _line(*parts):
    return " ".join(str(x) for p in parts for x in (p if isinstance(p, (list, tuple, np.ndarray)) else [p]))


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    d = tmp_path_factory.mktemp("svasan")
    exe = str(d / "sanitize_driver")
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", CSRC, os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "schedule.cpp"),
           os.path.join(NATIVE, "sanitize_driver.cpp"), "-o", exe]
    subprocess.run(cmd, check=True)
    return exe, d


def test_planner_and_schedule_clean_under_sanitizers(sanitized, planlib):
    exe, d = sanitized
    pcases, scases = _plan_cases(), _schedule_cases()
    lines = []
    for dims, par, pos, off, lens, kv, cap, target in pcases:
        lines.append(_line("P", dims, len(par), len(lens), kv, cap, target, par, pos, off, lens))
    acases = [([0] * 7, [0] * 12), ([0, 0, 8, 0, 0, 0, 0], [0] * 12), ([0] * 7, [0] * 11 + [2])]
    for w, n in acases:
        lines.append(_line("A", w, n))
    for n_cand, par, conf, rows, ms, cap in scases:
        lines.append(_line("S", len(n_cand), n_cand, par, conf, len(rows), rows, ms, cap))
    case_file = d / "cases.txt"
    case_file.write_text("\n".join(lines) + "\n")
    # (a library preloaded into every process by the environment may come
    # before the ASan runtime: the link-order check is off for that reason)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe, str(case_file)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    out = r.stdout.strip().split("\n")
    assert len(out) == len(lines)
    # the same statuses and plan figures as the plain build / the library
    from tests.test_host_abi import plan as plain_plan
    k = 0
    for dims, par, pos, off, lens, kv, cap, target in pcases:
        f = out[k].split()
        k += 1
        assert f[0] == "P"
        if len(dims) == 10 and dims[0] % dims[1] == 0 and dims[2] in (64, 128, 256):
            st, err, stats, anc, items = plain_plan(planlib, dims, par, pos, off, lens, kv, cap, target)
            assert int(f[1]) == st, (f, err)
            if st == 0:
                assert [int(x) for x in f[2:6]] == [int(stats[2]), int(stats[8]), int(stats[3]), int(stats[6])]
                assert int(f[6]) == int(sum(int(a) for a in anc[:len(par)])) % (1 << 64)
        else:
            assert int(f[1]) != 0
    for (w, n), want in zip(acases, [0, B.SV_ERR_INVALID_ARG, B.SV_ERR_INVALID_ARG]):
        assert out[k] == f"A {want}"
        k += 1
    for n_cand, par, conf, rows, ms, cap in scases:
        f = out[k].split()
        k += 1
        try:
            sel, tok, _ = B.spec_verify_schedule(n_cand, par, conf, rows, ms, cap)
            assert int(f[1]) == 0 and int(f[2]) == int(sel.sum()) and abs(float(f[3]) - tok) <= 1e-6 * max(1, tok)
        except B.SpecVerifyError as e:
            assert int(f[1]) == e.status
