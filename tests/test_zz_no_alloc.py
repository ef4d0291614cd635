"""The allocation-free entry point (spec_verify_run_static) against the
handle-based spec_verify_run on the same inputs, through the C ABI (needs an
MI355X): two calls in a row, the second with a smaller input, then a run
beyond its scratch capacity, refused with nothing enqueued."""
import numpy as np
import pytest

from draft_block_verification_verify_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from draft_block_verification_verify_amd import binding
    binding.lib()
    yield


def _static_run(dc, cfg, stream=None):
    import torch
    from draft_block_verification_verify_amd import binding as B
    s = stream if stream is not None else torch.cuda.current_stream().cuda_stream
    B.spec_verify_run_static(cfg, int(dc.w_o.data_ptr()), int(dc.w_lm.data_ptr()), dc.sv_in, dc.sv_out, s)


def _results(outs):
    import torch
    torch.cuda.synchronize()
    return {k: (v.cpu().numpy() if v is not None else None) for k, v in outs.items()}


def _same(a, b, what):
    # same kernels, same sizes, same order: identical results
    for k in a:
        if a[k] is None:
            continue
        np.testing.assert_array_equal(a[k], b[k], err_msg=f"{what}: {k}")


def _case(seed, n_roots_keep=None):
    """A chain-tiny (fp32) workload; optionally its first roots only."""
    cfg = W.CONFIGS[1]
    inp = W.make_inputs(cfg, seed)
    r = np.random.default_rng(seed)
    inp.draft_ids = r.integers(0, cfg.vocab, inp.st.n_rows).astype(np.int32)
    return inp


def test_static_entry_matches_the_handle_two_calls():
    from draft_block_verification_verify_amd import binding as B
    from draft_block_verification_verify_amd.runner import DeviceCase, sv_config
    # first call: the full tiny chain (8 rows), with a logits buffer
    inp = _case(0)
    dc = DeviceCase(inp, with_logits=True)
    try:
        dc.run()
        ref = dc.results()
        cfg = sv_config(inp.cfg, max_rows=inp.st.n_rows, max_roots=inp.st.n_roots, max_pos=int(inp.st.pos.max()) + 1)
        for v in dc.outs.values():
            if v is not None:
                v.fill_(-7)
        _static_run(dc, cfg)
        got = _results(dc.outs)
        _same(ref, got, "first call")
        assert (got["argmax"] >= 0).all()
    finally:
        dc.close()
    # second call right after: a smaller input (a 4-row chain on a shorter
    # prefix), no logits buffer (the logits then live in the scratch array)
    small = _case(1)
    small.st = W.chain_structure([37], 3)
    rows = np.arange(4)
    small.q_rows, small.k_rows, small.v_rows = small.q_rows[rows], small.k_rows[rows], small.v_rows[rows]
    small.kv_k, small.kv_v = small.kv_k[:37], small.kv_v[:37]
    small.drafter_logits = small.drafter_logits[:3]
    small.draft_ids = small.draft_ids[rows]
    dc2 = DeviceCase(small, with_logits=False)
    try:
        dc2.run()
        ref2 = dc2.results()
        cfg2 = sv_config(small.cfg, max_rows=4, max_roots=1, max_pos=int(small.st.pos.max()) + 1)
        for v in dc2.outs.values():
            if v is not None:
                v.fill_(-7)
        _static_run(dc2, cfg2)
        got2 = _results(dc2.outs)
        _same(ref2, got2, "second call")
        # the T = 1 mode through the same array
        ua, ub = W.make_uniforms(small)
        dc2.set_uniforms((ua, ub))
        dc2.run()
        ref3 = dc2.results()
        _static_run(dc2, cfg2)
        _same(ref3, _results(dc2.outs), "T = 1 call")
    finally:
        dc2.close()


def test_static_entry_refuses_what_it_cannot_hold():
    import torch
    from draft_block_verification_verify_amd import binding as B
    from draft_block_verification_verify_amd.runner import DeviceCase, sv_config
    inp = _case(2)
    dc = DeviceCase(inp, with_logits=False)
    try:
        for v in dc.outs.values():
            if v is not None:
                v.fill_(-7)
        # capacity: a vocabulary whose logits (8 rows x 300k x 4 B) overflow the 8 MiB array
        cfg = sv_config(inp.cfg, max_rows=inp.st.n_rows, max_roots=1, max_pos=int(inp.st.pos.max()) + 1)
        cfg.vocab = 300000
        with pytest.raises(B.SpecVerifyError) as e:
            _static_run(dc, cfg)
        assert e.value.status == B.SV_ERR_CAPACITY
        # bf16 models take the handle
        cfg = sv_config(inp.cfg, max_rows=inp.st.n_rows, max_roots=1, max_pos=int(inp.st.pos.max()) + 1)
        cfg.dtype = B.SV_BF16
        with pytest.raises(B.SpecVerifyError) as e:
            _static_run(dc, cfg)
        assert e.value.status == B.SV_ERR_UNSUPPORTED
        torch.cuda.synchronize()
        assert (dc.outs["argmax"] == -7).all() and (dc.outs["accept_len"] == -7).all()
    finally:
        dc.close()
