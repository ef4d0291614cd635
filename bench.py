#!/usr/bin/env python3
"""Throughput of one verify step on one MI355X.

A step is one spec_verify_run over one batch: RoPE + tree-masked GQA
attention + W_o + final norm + full-vocabulary LM head + vocab reductions +
overlaps + acceptance, metadata upload included.  Default workload: 32
concurrent chains at 27B shape (24/4 heads, d 256, hidden 5120, vocab
248,320), gamma 7 -> 256 verify rows, ragged bf16 KV prefixes
U{1024..16384}; synthetic seeded inputs, resident in HBM before timing.

Prints one JSON line (stdout).  Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verify rows/s (attn+LM-head+accept) γ=7, 27B shape; step ms; % of roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16/fp16 MFMA
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
# A GPU that has been idle (input generation takes seconds on the host) runs
# the first tens of milliseconds of load below its working clocks: before the
# warmup steps, the step runs untimed for at least this long.
SETTLE_S = 0.5
FLUSH_BYTES = 512 << 20        # written before each timed step (2x the 256 MB last-level cache)
COUNTERS = os.path.join(ROOT, "profiles", "lm_head_counters.json")
GEMM_SRC = [os.path.join(ROOT, "draft_block_verification_verify_amd", "csrc", f)
            for f in ("k_gemm.hip", "k_dma.hpp", "k_common.hpp", "launch.hpp")]   # launch.hpp: the blocked layout


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    """Hash of the sources the LM-head kernel is compiled from."""
    h = hashlib.sha256()
    for p in GEMM_SRC:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counters_traffic(workload: str):
    """HBM bytes per LM-head launch from committed rocprofv3 counter runs,
    if they were taken on this workload with the current kernel source."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    rec = c.get(workload)
    if not rec or rec.get("source_sha") != kernel_source_sha():
        return None
    return rec.get("bytes_per_launch")


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        return 1


def _oracle_sample(inp, cfg, d, roots, min_seconds: float):
    """The oracle on whole trees one after another until `min_seconds` of
    CPU work: (rows, trees, seconds)."""
    from oracle import verify_oracle as O
    rows, done, dt = 0, 0, 0.0
    t0 = time.perf_counter()
    while done < inp.st.n_roots and dt < min_seconds:
        O.verify(cfg, d, trees=[done])
        rows += int(roots[done + 1] - roots[done])
        done += 1
        dt = time.perf_counter() - t0
    return rows, done, dt


def cpu_baseline(inp, min_seconds: float = 6.0, fp8: bool = False, one_thread: bool = False) -> dict:
    """The fp64 oracle, as it stands, on the GPU machine's host: whole trees of
    the same workload one after another until at least `min_seconds` of CPU
    work (the sample), repeated for a median of 3 unless a run takes more than
    30 s; `one_thread` adds the same sample with BLAS limited to one thread.
    `fp8`: with the FP8 LM head."""
    from oracle import verify_oracle as O
    threads = _blas_threads()
    rng = np.random.default_rng(99)
    d = dict(O.inp_dict(inp))
    d["draft_ids"] = rng.integers(0, inp.cfg.vocab, inp.st.n_rows).astype(np.int32)
    roots = np.nonzero(inp.st.parent < 0)[0].tolist() + [inp.st.n_rows]
    cfg = O.cfg_dict(inp.cfg)
    if fp8:
        cfg["weight_format"] = "fp8"
    rows, done, dt = _oracle_sample(inp, cfg, d, roots, min_seconds)
    rates = [rows / dt]
    while len(rates) < 3 and dt <= 30.0:
        r2, _, dt2 = _fixed_sample(inp, cfg, d, roots, done)
        rates.append(r2 / dt2)
    kv = int(np.asarray(inp.st.root_kv_len)[:done].sum())
    out = {"value": float(np.median(rates)), "unit": "rows/s", "cores": int(threads), "kind": "oracle",
           "sample": f"trees 0..{done - 1} of {inp.st.n_roots} ({rows} rows, {kv} prefix tokens in all, "
                     f"full vocabulary), about {dt:.1f} s per run, median of {len(rates)} run(s)",
           "runs_rows_per_s": [float(x) for x in rates],
           "os_cpu_count": os.cpu_count(),
           "affinity_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
           "blas_threads": int(threads)}
    if one_thread:
        try:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1):
                r1, _, dt1 = _fixed_sample(inp, cfg, d, roots, done)
            out["one_thread"] = {"value": r1 / dt1, "unit": "rows/s", "cores": 1, "seconds": dt1}
        except Exception as e:          # threadpoolctl missing: say so
            out["one_thread"] = {"value": None, "error": str(e)}
    return out


def _fixed_sample(inp, cfg, d, roots, n_trees: int):
    """The oracle on trees 0 .. n_trees - 1: (rows, trees, seconds)."""
    from oracle import verify_oracle as O
    t0 = time.perf_counter()
    for t in range(n_trees):
        O.verify(cfg, d, trees=[t])
    return int(roots[n_trees] - roots[0]), n_trees, time.perf_counter() - t0


def copy_calibration(nbytes: int = 1 << 30, reps: int = 3) -> None:
    """A plain device copy of known size, for scaling HBM counters."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}))


def bench_rounds(args, cfg) -> int:
    """R chain decode steps: verify, commit the accepted paths into the KV
    cache, read the accept lengths back, lay out the next step (its roots
    after the committed rows; fresh seeded rows).  Drafts are planted on the
    target's greedy tokens by an untimed dry run of the same R steps; the
    timed replay must reproduce its accept lengths."""
    import torch
    from draft_block_verification_verify_amd import binding as B
    from draft_block_verification_verify_amd import workloads as W
    from draft_block_verification_verify_amd.runner import DeviceCase, to_device

    if cfg.kind == "tree":
        print("--rounds takes chain workloads (a shared stem cannot take commits)", file=sys.stderr)
        return 2
    R, gamma = args.rounds, cfg.gamma
    log(f"[rounds] generating {cfg.name} seed {args.seed}, {R} steps")
    inp = W.make_inputs(cfg, args.seed, slack=R * (gamma + 1))
    st = inp.st
    n, nd = st.n_rows, int((st.parent >= 0).sum())
    dc = DeviceCase(inp, max_pos=int(st.pos.max()) + 1 + R * (gamma + 1))
    dt = cfg.dtype
    rows = [{"q": dc.q, "k": dc.k, "v": dc.v, "dl": dc.dl}]
    for r in range(1, R):
        h = W.round_rows(cfg, args.seed, r, n, nd)
        rows.append({"q": to_device(h["q_rows"], dt, dc.device), "k": to_device(h["k_rows"], dt, dc.device),
                     "v": to_device(h["v_rows"], dt, dc.device), "dl": to_device(h["drafter_logits"], dt, dc.device)})
    kv0 = (dc.kv_k.clone(), dc.kv_v.clone())
    pos0, len0 = st.pos.copy(), st.root_kv_len.copy()

    # dry run: plant each step's drafts from the target's greedy tokens
    drafts, accs = [], []
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    commit_ms = []
    for r in range(R):
        if r:
            dc.next_step(accs[-1], rows[r])
        dc.run()
        W.plant_chain_drafts(inp, dc.results()["argmax"], rnd=r)
        dc.refresh()
        drafts.append(dc.draft_ids.clone())
        dc.run()
        ev[0].record()
        dc.commit()
        ev[1].record()
        accs.append(dc.results()["accept_len"].astype(np.int64))
        commit_ms.append(ev[0].elapsed_time(ev[1]))

    def reset():
        dc.kv_k.copy_(kv0[0])
        dc.kv_v.copy_(kv0[1])
        st.pos, st.root_kv_len = pos0.copy(), len0.copy()
        dc.q, dc.k, dc.v, dc.dl = rows[0]["q"], rows[0]["k"], rows[0]["v"], rows[0]["dl"]
        dc.draft_ids = drafts[0]
        dc.refresh(upload_drafts=False)
        torch.cuda.synchronize()

    def replay():
        got = []
        acc = None
        for r in range(R):
            if r:
                dc.next_step(acc, rows[r], drafts[r])
            dc.run()
            dc.commit()
            acc = dc.outs["accept_len"].cpu().numpy().astype(np.int64)   # the host waits here
            got.append(acc)
        return got

    settle(dc.run)
    reset()
    replay()                                   # warmup
    reset()
    log(f"[rounds] timing {R} steps")
    t0 = time.perf_counter()
    got = replay()
    torch.cuda.synchronize()
    t_loop = time.perf_counter() - t0
    replay_ok = all((a == b).all() for a, b in zip(got, accs))
    # the same steps' verify alone, back to back without commits or host waits
    reset()
    t0 = time.perf_counter()
    for _ in range(R):
        dc.run()
    torch.cuda.synchronize()
    t_verify = (time.perf_counter() - t0) / R
    dc.close()
    tokens = int(sum(a.sum() for a in got))
    res = {
        "metric": "decode tokens/s over R verify + commit steps (accepted drafts + bonus per sequence)",
        "value": tokens / t_loop,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": R,
        "warmup": 1,
        "ms_per_step": t_loop * 1e3 / R,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if dt == "bf16" else "f32",
        "data": "synthetic (seeded; random-init weights; drafts planted on the target's greedy tokens)",
        "config": {"workload": cfg.name, "sequences": st.n_roots, "gamma": gamma, "rounds": R, "seed": args.seed},
        "rounds": {"tokens": tokens, "accept_len_mean": float(np.mean([a.mean() for a in got])),
                   "verify_only_ms_per_step": t_verify * 1e3,
                   "fixed_cost_ms_per_step": t_loop * 1e3 / R - t_verify * 1e3,
                   "commit_kernel_ms_median": float(np.median(commit_ms)),
                   "replay_matches_dry_run": bool(replay_ok)},
    }
    print(json.dumps(res))
    return 0


def _sub_batch(W, inp, gam, drafts_full):
    """The chains' first gam[i] + 1 rows of a generated chain batch (same
    prefixes, same row tensors), with the full batch's draft ids."""
    import dataclasses
    st = inp.st
    roots = np.nonzero(st.parent < 0)[0]
    idx, parent = [], []
    for r, g in zip(roots, gam):
        s0 = len(idx)
        for j in range(int(g) + 1):
            idx.append(int(r) + j)
            parent.append(-1 if j == 0 else s0 + j - 1)
    idx = np.array(idx)
    draft_of = np.cumsum(st.parent >= 0) - 1          # draft-row number of each non-root row
    drows = [draft_of[i] for i in idx if st.parent[i] >= 0]
    sub_st = W.Structure(np.array(parent, np.int32), st.pos[idx].astype(np.int32), st.root_kv_off.copy(),
                         st.root_kv_len.copy(), st.kv_tokens)
    sub = dataclasses.replace(inp, st=sub_st, q_rows=inp.q_rows[idx], k_rows=inp.k_rows[idx],
                              v_rows=inp.v_rows[idx], drafter_logits=inp.drafter_logits[drows],
                              draft_ids=drafts_full[idx].astype(np.int32))
    return sub


def bench_schedule(args, cfg) -> int:
    """Verify budget over the concurrency batch: measure the step time of
    the batch at uniform gamma = 0..7 (the hardware curve), give request i a
    pass probability a_i ~ U(0.4, 0.95) per position and plant its drafts so
    that each next draft is accepted with probability a_i (draws fixed by the
    seed), then run, on the GPU, fixed-gamma batches and the scheduled
    ragged batch and count the tokens they commit per ms."""
    import torch
    from draft_block_verification_verify_amd import binding as B
    from draft_block_verification_verify_amd import workloads as W
    from draft_block_verification_verify_amd.runner import DeviceCase

    if cfg.kind != "multichain":
        print("--schedule takes the concurrency workload (--workload 5)", file=sys.stderr)
        return 2
    G = cfg.gamma
    inp = W.make_inputs(cfg, args.seed)
    st = inp.st
    R = st.n_roots
    full = DeviceCase(inp)
    full.run()
    greedy = full.results()["argmax"]
    # planted acceptance: k_i ~ truncated geometric with continuation a_i
    rng = np.random.default_rng([args.seed, 4242])
    a = rng.uniform(0.4, 0.95, R).astype(np.float32)
    ks = np.zeros(R, np.int64)
    for i in range(R):
        while ks[i] < G and rng.random() < a[i]:
            ks[i] += 1
    W.plant_chain_drafts(inp, greedy, k_per_tree=ks)
    drafts_full = inp.draft_ids.copy()
    kv = (full.kv_k, full.kv_v)
    weights = (full.w_o, full.w_lm)

    def timed(gam, steps):
        sub = _sub_batch(W, inp, gam, drafts_full)
        dc = DeviceCase(sub, verifier=full.ver, weights=weights, kv=kv)
        for _ in range(3):
            dc.run()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            dc.run()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        out = dc.results()
        return ms, int(out["accept_len"].sum()), sub.st.n_rows, out["accept_len"]

    settle(full.run)
    curve_g = [0, 1, 2, 3, 5, 7]
    curve = []
    for g in curve_g:
        ms, _, rows, _ = timed([g] * R, args.steps)
        curve.append((rows, ms))
        log(f"[schedule] gamma {g}: {rows} rows, {ms:.3f} ms")
    xs = [c[0] for c in curve]
    ys = list(np.maximum.accumulate(np.array([c[1] for c in curve], np.float32)))
    par = [j - 1 for _ in range(R) for j in range(G)]
    conf = [float(a[i]) for i in range(R) for _ in range(G)]
    sel, pred_tok, pred_ms = B.spec_verify_schedule([G] * R, par, conf, xs, ys)
    gam = sel.reshape(R, G).sum(axis=1)
    strategies = {}
    for name, gv in [("fixed_gamma_1", [1] * R), ("fixed_gamma_3", [3] * R), ("fixed_gamma_7", [G] * R),
                     ("scheduled", list(gam))]:
        ms, tok, rows, acc = timed(gv, args.steps)
        want = np.minimum(ks, np.asarray(gv)) + 1
        strategies[name] = {"rows": rows, "ms": ms, "tokens": tok, "tokens_per_ms": tok / ms,
                            "planted_ok": bool((acc == want).all())}
        log(f"[schedule] {name}: {rows} rows, {ms:.3f} ms, {tok} tokens")
    full.close()
    res = {
        "metric": "committed tokens per ms of one verify step, scheduled budget vs fixed gamma",
        "value": strategies["scheduled"]["tokens_per_ms"] * 1e3,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": 3,
        "ms_per_step": strategies["scheduled"]["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; per-request pass probabilities U(0.4, 0.95), planted acceptance)",
        "config": {"workload": cfg.name, "sequences": R, "max_gamma": G, "seed": args.seed},
        "schedule": {"curve_rows": xs, "curve_ms": [float(y) for y in ys], "gamma": [int(g) for g in gam],
                     "predicted_tokens": pred_tok, "predicted_ms": pred_ms, "strategies": strategies},
    }
    print(json.dumps(res))
    return 0


def settle(step) -> None:
    """Run `step` untimed, one at a time, for at least SETTLE_S seconds."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < SETTLE_S:
        step()
        torch.cuda.synchronize()
        n += 1
    log(f"[bench] settled: {n} untimed steps in {time.perf_counter() - t0:.2f} s")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--workload", type=int, default=5, choices=[1, 2, 3, 4, 5],
                    help="1 chain-tiny, 2 chain-8b, 3 block-27b-b16, 4 tree-specopd, 5 conc32-27b (default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", dest="other_configs", action="store_false",
                    help="measure only --workload (by default the other four configurations follow, "
                         "reported under other_configs)")
    ap.add_argument("--sample", action="store_true",
                    help="T = 1 stochastic verification (drafts drawn from the drafter, seeded uniforms)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--fp8", action="store_true",
                    help="FP8 (e4m3, W8A8) LM head (bf16 workloads)")
    ap.add_argument("--schedule", action="store_true",
                    help="conc32: measure the rows -> ms curve, then compare fixed gamma with the verify-budget "
                         "schedule on synthetic per-request confidences")
    ap.add_argument("--rounds", type=int, default=0,
                    help="chain workloads: time R decode steps of verify + commit (host reads the accept "
                         "lengths each step) instead of the single verify step")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the verify step here is "
              "a single-GPU implementation with no sharding across GPUs", file=sys.stderr)
        return 2
    import torch
    if args.copy_calibration:
        copy_calibration()
        return 0

    from draft_block_verification_verify_amd import binding as B
    from draft_block_verification_verify_amd import workloads as W

    B.lib()                                   # fails loudly without the HIP library
    cfg = W.CONFIGS[args.workload]
    if args.rounds:
        return bench_rounds(args, cfg)
    if args.schedule:
        return bench_schedule(args, cfg)
    peaks = measured_peaks()
    log(f"[bench] measured peaks: copy {peaks['copy_gbs']:.0f} GB/s, bf16 GEMM {peaks['gemm_bf16_tflops']:.0f} TFLOP/s")
    head = measure(cfg, args.seed, args.steps, args.warmup, fp8=args.fp8, sample=args.sample, peaks=peaks,
                   cpu=not args.no_cpu_baseline, stages=True)
    res = {
        "metric": METRIC,
        "value": head["rows_per_s"],
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_p50"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16, LM head e4m3" if args.fp8 else "bf16") if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; random-init weights of the stated shapes)",
        "config": head["config"],
        "roofline": head["roofline"],
        "timing": head["timing"],
        "step": head["step"],
        "measured_peaks": peaks,
        "cpu_baseline": head.get("cpu_baseline"),
    }
    if args.other_configs and not (args.fp8 or args.sample):
        # every other configuration in the same run, same protocol, fewer steps
        others = {}
        for wid in (1, 2, 3, 4):
            if wid == args.workload:
                continue
            c = W.CONFIGS[wid]
            o = measure(c, args.seed, max(5, args.steps // 2), 3, peaks=peaks, cpu=not args.no_cpu_baseline,
                        one_thread=wid <= 3)
            others[c.name] = {k: o[k] for k in ("rows_per_s", "ms_p50", "config", "roofline", "timing", "step",
                                                "cpu_baseline") if k in o}
        res["other_configs"] = others
    print(json.dumps(res))
    return 0


def measured_peaks() -> dict:
    """Achievable peaks measured on this GPU, beside the nominal ones: a
    1 GiB device-to-device copy (bytes read + written per second, best of 5)
    and a dense 8192^3 bf16 GEMM (torch.mm, best of 5)."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    src.fill_(3)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    best = float("inf")
    for _ in range(6):
        ev[0].record()
        dst.copy_(src)
        ev[1].record()
        torch.cuda.synchronize()
        best = min(best, ev[0].elapsed_time(ev[1]))
    copy_gbs = 2 * n / (best * 1e-3) / 1e9
    del src, dst
    m = 8192
    a = torch.randn(m, m, dtype=torch.bfloat16, device="cuda:0")
    b = torch.randn(m, m, dtype=torch.bfloat16, device="cuda:0")
    for _ in range(3):
        torch.mm(a, b)
    best = float("inf")
    for _ in range(5):
        ev[0].record()
        torch.mm(a, b)
        ev[1].record()
        torch.cuda.synchronize()
        best = min(best, ev[0].elapsed_time(ev[1]))
    del a, b
    torch.cuda.empty_cache()
    return {"copy_gbs": copy_gbs, "gemm_bf16_tflops": 2 * m ** 3 / (best * 1e-3) / 1e12,
            "copy": "1 GiB device-to-device copy, read + write bytes, best of 6",
            "gemm": "torch.mm bf16 8192 x 8192 x 8192, best of 5 after 3"}


class Flusher:
    """Writes FLUSH_BYTES (twice the 256 MB last-level cache) on the current
    stream before each timed step, outside the timed interval, so that the
    weights and the KV cache come from HBM as in a step of a deep model."""

    def __init__(self):
        import torch
        self.buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda:0")
        self.i = 0

    def __call__(self):
        self.i += 1
        self.buf.fill_(self.i & 0xFF)


def timed_steps(step, steps: int, flush) -> np.ndarray:
    """Per-step device times (ms) by two HIP events on the step's stream (the
    current stream), a cache flush before each step outside its events."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in evs:
        flush()
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in evs])


def measure(cfg, seed, steps, warmup, *, fp8=False, sample=False, peaks=None, cpu=True, one_thread=False,
            stages=False) -> dict:
    """One workload: inputs resident in HBM, drafts planted, then the timed
    steps (profiling off), the LM-head loop (its launch between two events),
    and optionally the per-stage loop and the oracle on the host."""
    import torch
    from draft_block_verification_verify_amd import accounting as A
    from draft_block_verification_verify_amd import binding as B
    from draft_block_verification_verify_amd import workloads as W
    from draft_block_verification_verify_amd.runner import DeviceCase

    log(f"[bench] generating {cfg.name} seed {seed}")
    t0 = time.perf_counter()
    inp = W.make_inputs(cfg, seed)
    st = inp.st
    log(f"[bench] inputs ready in {time.perf_counter() - t0:.1f} s: rows {st.n_rows}, trees {st.n_roots}, "
        f"kv tokens {st.kv_tokens}")
    dc = DeviceCase(inp, with_logits=False, fp8=fp8)
    torch.cuda.synchronize()

    # draft ids: trees use draws from the drafter; chains get a planted
    # accepted prefix k ~ U{0..gamma} on the target's greedy tokens (taken from
    # a first run of this same step)
    planted = None
    if cfg.kind == "tree" or sample:
        W.sample_tree_drafts(inp)
    else:
        dc.run()
        planted = W.plant_chain_drafts(inp, dc.results()["argmax"])
    if sample:
        dc.set_uniforms(W.make_uniforms(inp))
    dc.refresh()
    flush = Flusher()

    settle(dc.run)
    log(f"[bench] {cfg.name}: warmup {warmup}")
    for _ in range(warmup):
        flush()
        dc.run()
    torch.cuda.synchronize()
    # the timed steps, profiling off
    log(f"[bench] {cfg.name}: timing {steps} steps")
    t0 = time.perf_counter()
    step_ms = timed_steps(dc.run, steps, flush)
    wall = time.perf_counter() - t0
    out = dc.results()
    ok = bool((out["accept_len"] == planted + 1).all()) if planted is not None else None
    # the LM-head launch between two events, same protocol
    B.spec_verify_profile(dc.ver.h, 2)
    lm_step_ms = timed_steps(dc.run, steps, flush)
    lm_ms = dict(B.spec_verify_stage_times(dc.ver.h)).get("lm_head", float("nan"))
    B.spec_verify_profile(dc.ver.h, 0)
    stage_ms = {}
    if stages:
        # events around every stage (they add a few microseconds each)
        B.spec_verify_profile(dc.ver.h, 1)
        timed_steps(dc.run, steps, flush)
        stage_ms = dict(B.spec_verify_stage_times(dc.ver.h))
        B.spec_verify_profile(dc.ver.h, 0)
    dc.close()

    n = st.n_rows
    p10, p50, p90 = (float(x) for x in np.percentile(step_ms, [10, 50, 90]))
    sb, sf = A.step_bytes(cfg, st, fp8=fp8), A.step_flops(cfg, st)
    mfma_peak = FP8_PEAK_TFLOPS if fp8 else BF16_PEAK_TFLOPS
    lm_bytes, lm_flops = sb["lm_head"], sf["lm_head"]
    ridge = mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    meas_bw = peaks["copy_gbs"] if peaks else None
    meas_mfma = None if (fp8 or not peaks) else peaks["gemm_bf16_tflops"]
    if lm_flops / lm_bytes < ridge:
        achieved = lm_bytes / (lm_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS,
                "measured_peak": meas_bw, "frac_of_measured": achieved / meas_bw if meas_bw else None}
    else:
        achieved = lm_flops / (lm_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": mfma_peak, "unit": "TFLOP/s",
                "frac": achieved / mfma_peak,
                "measured_peak": meas_mfma, "frac_of_measured": achieved / meas_mfma if meas_mfma else None}
    roof["traffic"] = None if fp8 else counters_traffic(cfg.name)
    roof.update(kernel="lm_head", kernel_ms=lm_ms, algorithmic_bytes=lm_bytes, algorithmic_flops=lm_flops,
                mfma_frac=lm_flops / (lm_ms * 1e-3) / 1e12 / mfma_peak,
                hbm_frac=lm_bytes / (lm_ms * 1e-3) / 1e9 / HBM_PEAK_GBS)
    step_s = p50 * 1e-3
    res = {
        "rows_per_s": n / step_s,
        "ms_p50": p50,
        "config": {"workload": cfg.name, "rows": n, "trees": st.n_roots, "kv_tokens": int(st.kv_tokens),
                   "heads_q_kv": [cfg.n_q_heads, cfg.n_kv_heads], "head_dim": cfg.head_dim,
                   "hidden": cfg.hidden, "vocab": cfg.vocab, "gamma": cfg.gamma, "seed": seed,
                   "dtype": cfg.dtype, "acceptance": "T=1 sampling" if sample else "greedy",
                   "lm_head_format": "fp8 e4m3 (W8A8)" if fp8 else "native"},
        "roofline": roof,
        "timing": {"ms_p10": p10, "ms_p50": p50, "ms_p90": p90, "ms_mean": float(step_ms.mean()),
                   "steps": int(steps), "flush_bytes_before_each_step": FLUSH_BYTES,
                   "events": "two HIP events on the run's stream around each step, profiling off",
                   "wall_s_timed_loop": wall,
                   "lm_head_loop_step_ms_p50": float(np.median(lm_step_ms))},
        "step": {"algorithmic_bytes": sb["total"], "algorithmic_flops": sf["total"],
                 "hbm_frac_of_step": sb["total"] / step_s / 1e9 / HBM_PEAK_GBS,
                 "hbm_frac_of_step_measured_peak": (sb["total"] / step_s / 1e9 / meas_bw) if meas_bw else None,
                 "stages_ms": {k: v for k, v in stage_ms.items() if k != "step"},
                 "device_ms_staged": stage_ms.get("step"),
                 "planted_accept_ok": ok,
                 "accept_len_mean": float(out["accept_len"].mean())},
    }
    if cpu:
        log(f"[bench] {cfg.name}: cpu baseline (the oracle on whole sequences)")
        res["cpu_baseline"] = cpu_baseline(inp, fp8=fp8, one_thread=one_thread)
    else:
        res["cpu_baseline"] = None
    del dc, inp, flush
    torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    sys.exit(main())
