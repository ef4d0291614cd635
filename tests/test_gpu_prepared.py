"""Prepared weights (spec_verify_prepare_weights, spec_verify_create_prepared)
against a handle that converts the same bf16 weights itself (needs an
MI355X).  Both run the same kernels on the same fp16 values, so every output
must be bit-identical; two handles may share one prepared buffer, and a
weight outside the fp16 range is refused as spec_verify_create refuses it.
"""
import dataclasses

import numpy as np
import pytest

from draft_block_verification_verify_amd import workloads as W
from tests.test_gpu_parity import MINIS, _say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from draft_block_verification_verify_amd import binding
    binding.lib()          # fails loudly if the HIP library is missing
    yield


def _inputs(name, seed=0):
    cfg = MINIS[name]
    inp = W.make_inputs(cfg, seed)
    if cfg.kind == "tree":
        W.sample_tree_drafts(inp)
    return inp


def _run(inp, verifier=None, max_rows=None):
    from draft_block_verification_verify_amd.runner import DeviceCase
    dc = DeviceCase(inp, with_logits=True, verifier=verifier, max_rows=max_rows)
    try:
        dc.run()
        return dc.results()
    finally:
        dc.close()


def _prepared_verifier(inp, buf=None, extra_rows=0):
    import torch
    from draft_block_verification_verify_amd import binding as B
    from draft_block_verification_verify_amd import runner as R
    st = inp.st
    svc = R.sv_config(inp.cfg, max_rows=st.n_rows + extra_rows, max_roots=st.n_roots, max_pos=int(st.pos.max()) + 1)
    w_o = R.to_device(inp.w_o, "bf16", "cuda:0")
    w_lm = R.to_device(inp.w_lm, "bf16", "cuda:0")
    if buf is None:
        buf = torch.empty(B.spec_verify_weight_bytes(svc), dtype=torch.uint8, device="cuda:0")
        assert buf.data_ptr() % 256 == 0
        B.spec_verify_prepare_weights(svc, w_o.data_ptr(), w_lm.data_ptr(), buf.data_ptr())
    return B.Verifier(svc, None, None, prepared=buf), buf


@pytest.mark.parametrize("name", ["c2m", "c4m", "c5m", "c5t"])
def test_prepared_weights_match_the_copying_handle(name):
    inp = _inputs(name)
    _say(f"[prepared] {name} rows={inp.st.n_rows}")
    ref = _run(inp)
    ver, buf = _prepared_verifier(inp)
    got = _run(inp, verifier=ver)
    for k in ref:
        np.testing.assert_array_equal(got[k], ref[k], err_msg=k)
    # a second handle with larger capacities borrowing the same buffer,
    # against a copying handle of those capacities (the capacities can
    # change the attention work split, so the reference changes with them)
    ref2 = _run(inp, max_rows=inp.st.n_rows + 40)
    ver2, _ = _prepared_verifier(inp, buf, extra_rows=40)
    got2 = _run(inp, verifier=ver2)
    for k in ref2:
        np.testing.assert_array_equal(got2[k], ref2[k], err_msg=k)


def test_prepare_refuses_weights_outside_fp16():
    from draft_block_verification_verify_amd import binding as B
    inp = _inputs("c2m")
    w_lm = np.array(inp.w_lm, copy=True)
    # bf16 bit pattern of 2^17 (outside the fp16 range)
    w_lm.reshape(-1)[5] = np.uint16(0x4800)
    bad = dataclasses.replace(inp, w_lm=w_lm)
    with pytest.raises(B.SpecVerifyError) as e:
        _prepared_verifier(bad)
    assert "fp16 range" in str(e.value) or "65504" in str(e.value)
    assert B.spec_verify_last_error()
