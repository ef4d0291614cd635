"""The tiled LM head's K-loop protocol on the CPU: a model of every wave's
sequence of DMA issues, DMA waits, barriers and LDS reads, for the plain
loop and for the ping-pong loop (waves 4-7 one barrier behind waves 0-3),
checked for

* equal barrier counts in every wave (a mismatch hangs the workgroup);
* every read of stage s after every wave's wait for its share of stage s,
  ordered through a barrier;
* every refill of a ring slot after every wave's reads of the stage that
  slot held, ordered through a barrier (or program order in the same wave).

The schedule mirrors gemm_tiled_kernel in k_gemm.hip: ST - 1 stages issued
before the first step; at step s a wait that leaves `younger` of the wave's
own stages in flight, then the barrier, the issue of stage s + ST - 1, the
fragment reads of stage s; in the ping-pong loop an LDS drain and a second
barrier before the MFMAs, the lagging group's extra barrier (after its wait
for stage 0) before the first step, the leading group's after the last.
Two planted mistakes must fail the checks.
"""
import pytest

W = 8


def wave_ops(lag, pp, st, nk, tiles, drop_stage0_wait=False, drain_after_barrier=False):
    ops = []

    def wait_then_barrier(younger):
        ops.append(("wait", younger))
        ops.append(("bar",))

    for t in range(tiles):
        base = t * 1000
        for p in range(st - 1):
            if p < nk:
                ops.append(("issue", base + p))
        if pp and lag:
            if drop_stage0_wait:
                ops.append(("bar",))
            else:
                wait_then_barrier(min(st - 2, nk - 1))
        for s in range(nk):
            younger = max(0, min(st - 3, nk - 2 - s)) if (pp and lag) else min(st - 2, nk - 1 - s)
            wait_then_barrier(younger)
            if s + st - 1 < nk:
                ops.append(("issue", base + s + st - 1))
            ops.append(("read", base + s))
            if pp and drain_after_barrier:
                ops.append(("bar",))
                ops.append(("done", base + s))
            elif pp:
                ops.append(("done", base + s))
                ops.append(("bar",))
            else:
                ops.append(("done", base + s))   # the MFMAs consume the fragments before the next barrier
        if pp and not lag:
            ops.append(("bar",))
        ops.append(("bar",))   # epilogue: every wave is done reading the ring
        ops.append(("bar",))   # the statistics exchange
    return ops


def check(pp, st, nk, tiles=3, **plant):
    waves = [wave_ops(w >= 4, pp, st, nk, tiles, **plant) for w in range(W)]
    counts = {sum(1 for o in ops if o[0] == "bar") for ops in waves}
    assert len(counts) == 1, "barrier counts differ"
    info = []
    for ops in waves:
        issued, bars = [], 0
        landed, read, done, issue = {}, {}, {}, {}
        for op in ops:
            kind = op[0]
            if kind == "issue":
                issued.append(op[1])
                issue[op[1]] = bars
            elif kind == "wait":
                y = op[1]
                for k in (issued[:len(issued) - y] if y else issued):
                    landed.setdefault(k, bars)   # landed before barrier number bars + 1
            elif kind == "bar":
                bars += 1
            elif kind == "read":
                assert op[1] in landed, "a wave reads its own stage before waiting for it"
                read[op[1]] = bars
            elif kind == "done":
                done[op[1]] = bars
        info.append((landed, read, done, issue))
    for j, (_, read_j, _, issue_j) in enumerate(info):
        for s, bj in read_j.items():
            for i, (landed_i, _, _, _) in enumerate(info):
                if i != j:
                    assert s in landed_i and landed_i[s] + 1 <= bj, ("read before landed", j, i, s)
        for k, bj in issue_j.items():
            slot = (k % 1000) % st
            for i, (_, _, done_i, _) in enumerate(info):
                for s, bi in done_i.items():
                    same_slot = s // 1000 == k // 1000 and s < k and (s % 1000) % st == slot
                    earlier_tile = s // 1000 < k // 1000
                    if not (same_slot or earlier_tile):
                        continue
                    if i == j:
                        assert bi <= bj, ("refill before own read", j, k, s)
                    else:
                        assert bi + 1 <= bj, ("refill before read done", j, i, k, s)


@pytest.mark.parametrize("pp", [False, True])
@pytest.mark.parametrize("st", [3, 4, 5])
@pytest.mark.parametrize("nk", [1, 2, 3, 4, 5, 8, 17])
def test_protocol_holds(pp, st, nk):
    check(pp, st, nk)


def test_missing_stage0_wait_is_caught():
    with pytest.raises(AssertionError, match="read before landed"):
        check(True, 4, 8, drop_stage0_wait=True)


def test_missing_drain_before_the_mid_barrier_is_caught():
    with pytest.raises(AssertionError, match="refill before"):
        for st in (3, 4):
            check(True, st, 8, drain_after_barrier=True)
