"""Device plumbing around the C ABI: upload a generated workload with torch,
create a handle, run the verify step, read the outputs back.

Nothing here computes any part of the verify step.
"""
from __future__ import annotations

import numpy as np

from . import binding as B
from .workloads import Config, Inputs


def sv_config(cfg: Config, *, max_rows: int, max_roots: int, max_tree_rows: int = 64,
              max_pos: int = 1 << 20, fp8: bool = False) -> B.SvConfig:
    return B.SvConfig(cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.hidden, cfg.vocab,
                      B.SV_BF16 if cfg.dtype == "bf16" else B.SV_F32, cfg.rope_base, cfg.norm_eps,
                      max_rows, max_roots, max_tree_rows, max_pos,
                      B.SV_WEIGHTS_FP8 if fp8 else B.SV_WEIGHTS_NATIVE)


def to_device(x: np.ndarray | None, dtype: str, device):
    import torch
    if x is None:
        return None
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16))
        return t.to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


class DeviceCase:
    """A workload resident on the GPU plus a handle ready to run it."""

    def __init__(self, inp: Inputs, device="cuda:0", *, with_logits: bool = False, verifier=None,
                 weights=None, max_rows: int | None = None, max_roots: int | None = None,
                 uniforms=None, max_pos: int | None = None, kv=None, fp8: bool = False):
        import torch
        self.inp = inp
        cfg, st = inp.cfg, inp.st
        self.device = torch.device(device)
        dt = cfg.dtype
        if kv is not None:                    # the cache already on the device (shared)
            self.kv_k, self.kv_v = kv
        else:
            self.kv_k = to_device(inp.kv_k, dt, device) if st.kv_tokens > 0 else None
            self.kv_v = to_device(inp.kv_v, dt, device) if st.kv_tokens > 0 else None
        self.q = to_device(inp.q_rows, dt, device)
        self.k = to_device(inp.k_rows, dt, device)
        self.v = to_device(inp.v_rows, dt, device)
        self.dl = to_device(inp.drafter_logits, dt, device) if inp.drafter_logits.shape[0] else None
        self.draft_ids = torch.from_numpy(np.ascontiguousarray(inp.draft_ids, np.int32)).to(device)
        if weights is None:
            weights = (to_device(inp.w_o, dt, device), to_device(inp.w_lm, dt, device))
        self.w_o, self.w_lm = weights
        if verifier is None:
            verifier = B.Verifier(sv_config(cfg, max_rows=max_rows or st.n_rows,
                                            max_roots=max_roots or st.n_roots,
                                            max_pos=max_pos or int(st.pos.max()) + 1, fp8=fp8),
                                  self.w_o, self.w_lm)
        self.ver = verifier
        self.outs = verifier.alloc_outputs(st.n_rows, st.n_roots, self.device, with_logits)
        self.set_uniforms(uniforms)

    def set_uniforms(self, uniforms):
        """(u_accept, u_bonus) host arrays switch the runs to T = 1 stochastic
        verification; None switches back to greedy."""
        import torch
        if uniforms is None:
            self.u_accept = self.u_bonus = None
        else:
            self.u_accept = torch.from_numpy(np.ascontiguousarray(uniforms[0], np.float32)).to(self.device)
            self.u_bonus = torch.from_numpy(np.ascontiguousarray(uniforms[1], np.float32)).to(self.device)
        self.refresh()

    def refresh(self, upload_drafts: bool = True):
        """Rebuild the C structs (after draft ids or structure change)."""
        import torch
        st = self.inp.st
        if upload_drafts:
            self.draft_ids = torch.from_numpy(np.ascontiguousarray(self.inp.draft_ids, np.int32)).to(self.device)
        self.sv_in, self.sv_out, self._keep = B.Verifier.make_structs(
            st.parent, st.pos, st.root_kv_off, st.root_kv_len, self.kv_k, self.kv_v, self.q, self.k,
            self.v, self.draft_ids, self.dl, self.outs,
            B.SV_MODE_SAMPLE if self.u_accept is not None else B.SV_MODE_GREEDY, self.u_accept, self.u_bonus)
        if self.kv_k is None:
            self.sv_in.kv_tokens = 0

    def run(self, stream=None):
        import torch
        s = stream if stream is not None else torch.cuda.current_stream(self.device).cuda_stream
        self.ver.run(self.sv_in, self.sv_out, s)

    def commit(self, stream=None):
        """Enqueue the commit of the last run (accepted paths into the cache)."""
        import torch
        s = stream if stream is not None else torch.cuda.current_stream(self.device).cuda_stream
        self.ver.commit(self.sv_in, self.sv_out, self.kv_k, self.kv_v, s)

    def next_step(self, accept_len, rows=None, draft_ids=None):
        """Lay out the next chain step after a commit: each tree keeps its
        cache segment and sees accept_len more entries, and its rows move
        accept_len positions on (the new root follows the last committed
        row).  `rows` replaces the row tensors: a dict of host arrays
        (q_rows, k_rows, v_rows, drafter_logits) or of device tensors
        (q, k, v, dl).  Draft ids: `draft_ids` (host or device int32) or
        zeros."""
        import torch
        st = self.inp.st
        acc = np.asarray(accept_len, np.int64)
        roots = np.nonzero(st.parent < 0)[0]
        ends = list(roots[1:]) + [st.n_rows]
        pos = st.pos.astype(np.int64)
        for t, (a, b) in enumerate(zip(roots, ends)):
            pos[a:b] += acc[t]
        st.pos = pos.astype(np.int32)
        st.root_kv_len = (st.root_kv_len.astype(np.int64) + acc).astype(np.int32)
        if rows is not None:
            dt = self.inp.cfg.dtype
            if "q" in rows:
                self.q, self.k, self.v, self.dl = rows["q"], rows["k"], rows["v"], rows["dl"]
            else:
                self.q = to_device(rows["q_rows"], dt, self.device)
                self.k = to_device(rows["k_rows"], dt, self.device)
                self.v = to_device(rows["v_rows"], dt, self.device)
                self.dl = to_device(rows["drafter_logits"], dt, self.device)
                self.inp.q_rows, self.inp.k_rows = rows["q_rows"], rows["k_rows"]
                self.inp.v_rows, self.inp.drafter_logits = rows["v_rows"], rows["drafter_logits"]
        on_device = draft_ids is not None and not isinstance(draft_ids, np.ndarray)
        if draft_ids is None:
            self.inp.draft_ids = np.zeros(st.n_rows, np.int32)
        elif not on_device:
            self.inp.draft_ids = draft_ids.astype(np.int32)
        else:
            self.draft_ids = draft_ids
        self.refresh(upload_drafts=not on_device)

    def results(self) -> dict:
        import torch
        torch.cuda.synchronize(self.device)
        return {k: (v.cpu().numpy() if v is not None else None) for k, v in self.outs.items()}

    def close(self):
        self.ver.close()
