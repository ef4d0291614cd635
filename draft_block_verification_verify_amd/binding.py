"""ctypes binding of libspecverify.so (C ABI in include/spec_verify.h).

Argument marshalling only: every step of the verify computation runs in the
HIP library.  torch is used for device memory and streams.  Loading fails
loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_lib", "libspecverify.so")

SV_OK, SV_ERR_INVALID_ARG, SV_ERR_BAD_TREE, SV_ERR_CAPACITY = 0, -1, -2, -3
SV_ERR_UNSUPPORTED, SV_ERR_HIP, SV_ERR_OOM = -4, -5, -6
SV_F32, SV_BF16 = 0, 1
SV_WEIGHTS_NATIVE, SV_WEIGHTS_FP8 = 0, 1
STATUS_NAMES = {0: "SV_OK", -1: "SV_ERR_INVALID_ARG", -2: "SV_ERR_BAD_TREE", -3: "SV_ERR_CAPACITY",
                -4: "SV_ERR_UNSUPPORTED", -5: "SV_ERR_HIP", -6: "SV_ERR_OOM"}


class SvConfig(C.Structure):
    _fields_ = [("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("hidden", C.c_int32), ("vocab", C.c_int32), ("dtype", C.c_int32),
                ("rope_base", C.c_float), ("norm_eps", C.c_float),
                ("max_rows", C.c_int32), ("max_roots", C.c_int32), ("max_tree_rows", C.c_int32),
                ("max_pos", C.c_int32), ("weight_format", C.c_int32)]


class SvInputs(C.Structure):
    _fields_ = [("n_rows", C.c_int32), ("n_roots", C.c_int32),
                ("parent", C.POINTER(C.c_int32)), ("pos", C.POINTER(C.c_int32)),
                ("root_kv_off", C.POINTER(C.c_int64)), ("root_kv_len", C.POINTER(C.c_int32)),
                ("kv_tokens", C.c_int64),
                ("kv_k", C.c_void_p), ("kv_v", C.c_void_p),
                ("q_rows", C.c_void_p), ("k_rows", C.c_void_p), ("v_rows", C.c_void_p),
                ("draft_ids", C.c_void_p), ("drafter_logits", C.c_void_p),
                ("mode", C.c_int32), ("u_accept", C.c_void_p), ("u_bonus", C.c_void_p)]


SV_MODE_GREEDY, SV_MODE_SAMPLE = 0, 1


class SvOutputs(C.Structure):
    _fields_ = [("accept_len", C.c_void_p), ("bonus", C.c_void_p), ("last_row", C.c_void_p),
                ("surv_sum", C.c_void_p), ("argmax", C.c_void_p), ("row_max", C.c_void_p),
                ("row_lse", C.c_void_p), ("overlap", C.c_void_p), ("survival", C.c_void_p),
                ("logits", C.c_void_p)]


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_lib = None

# exported symbols and their signatures (checked by the CPU tests)
SYMBOLS = {
    "spec_verify_create": (C.c_int, [C.POINTER(SvConfig), C.c_void_p, C.c_void_p, C.POINTER(C.c_void_p)]),
    "spec_verify_run": (C.c_int, [C.c_void_p, C.POINTER(SvInputs), C.POINTER(SvOutputs), C.c_void_p]),
    "spec_verify_commit": (C.c_int, [C.c_void_p, C.POINTER(SvInputs), C.POINTER(SvOutputs), C.c_void_p, C.c_void_p,
                                     C.c_void_p]),
    "spec_verify_schedule": (C.c_int, [C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p,
                                       C.c_void_p, C.c_int32, C.c_void_p, C.POINTER(C.c_double),
                                       C.POINTER(C.c_double)]),
    "spec_verify_run_static": (C.c_int, [C.POINTER(SvConfig), C.c_void_p, C.c_void_p, C.POINTER(SvInputs),
                                         C.POINTER(SvOutputs), C.c_void_p]),
    "spec_verify_weight_bytes": (C.c_int, [C.POINTER(SvConfig), C.POINTER(C.c_size_t)]),
    "spec_verify_prepare_weights": (C.c_int, [C.POINTER(SvConfig), C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]),
    "spec_verify_create_prepared": (C.c_int, [C.POINTER(SvConfig), C.c_void_p, C.POINTER(C.c_void_p)]),
    "spec_verify_destroy": (C.c_int, [C.c_void_p]),
    "spec_verify_last_error": (C.c_char_p, []),
    "spec_verify_profile": (C.c_int, [C.c_void_p, C.c_int32]),
    "spec_verify_stage_times": (C.c_int32, [C.c_void_p, C.POINTER(C.c_char_p), C.POINTER(C.c_float), C.c_int32]),
}


def lib(path: str | None = None):
    """Load the HIP library (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"HIP library not built: {p} is missing "
                           "(run `python -m draft_block_verification_verify_amd.build`)")
    L = C.CDLL(p)
    for name, (res, args) in SYMBOLS.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def spec_verify_last_error() -> str:
    return lib().spec_verify_last_error().decode()


def _check(st: int):
    if st != SV_OK:
        raise SpecVerifyError(st, spec_verify_last_error())


def spec_verify_create(cfg: SvConfig, w_o_ptr: int, w_lm_ptr: int) -> C.c_void_p:
    h = C.c_void_p()
    _check(lib().spec_verify_create(C.byref(cfg), C.c_void_p(w_o_ptr), C.c_void_p(w_lm_ptr), C.byref(h)))
    return h


def spec_verify_weight_bytes(cfg: SvConfig) -> int:
    n = C.c_size_t(0)
    _check(lib().spec_verify_weight_bytes(C.byref(cfg), C.byref(n)))
    return int(n.value)


def spec_verify_prepare_weights(cfg: SvConfig, w_o_ptr: int, w_lm_ptr: int, dst_ptr: int,
                                stream: int | None = None) -> None:
    _check(lib().spec_verify_prepare_weights(C.byref(cfg), C.c_void_p(w_o_ptr), C.c_void_p(w_lm_ptr),
                                             C.c_void_p(dst_ptr), C.c_void_p(stream or 0)))


def spec_verify_create_prepared(cfg: SvConfig, prepared_ptr: int) -> C.c_void_p:
    h = C.c_void_p()
    _check(lib().spec_verify_create_prepared(C.byref(cfg), C.c_void_p(prepared_ptr), C.byref(h)))
    return h


def spec_verify_run(h, inputs: SvInputs, outputs: SvOutputs, stream: int | None = None) -> None:
    _check(lib().spec_verify_run(h, C.byref(inputs), C.byref(outputs), C.c_void_p(stream or 0)))


def spec_verify_commit(h, inputs: SvInputs, outputs: SvOutputs, kv_k: int, kv_v: int,
                       stream: int | None = None) -> None:
    _check(lib().spec_verify_commit(h, C.byref(inputs), C.byref(outputs), C.c_void_p(kv_k), C.c_void_p(kv_v),
                                    C.c_void_p(stream or 0)))


def spec_verify_schedule(n_cand, cand_parent, cand_conf, curve_rows, curve_ms, max_rows: int = 0):
    """Host-only budget schedule (see spec_verify.h).  Candidate arrays are
    the requests' candidates one after another.  Returns (selected int32
    array, expected tokens, step ms)."""
    n_cand = host_i32(n_cand)
    par = host_i32(cand_parent)
    conf = np.ascontiguousarray(np.asarray(cand_conf, dtype=np.float32))
    cr = host_i32(curve_rows)
    cm = np.ascontiguousarray(np.asarray(curve_ms, dtype=np.float32))
    sel = np.zeros(max(int(n_cand.sum()), 1), np.int32)
    tok, ms = C.c_double(), C.c_double()
    _check(lib().spec_verify_schedule(int(n_cand.shape[0]), n_cand.ctypes.data, par.ctypes.data, conf.ctypes.data,
                                      int(cr.shape[0]), cr.ctypes.data, cm.ctypes.data, int(max_rows),
                                      sel.ctypes.data, C.byref(tok), C.byref(ms)))
    return sel[:int(n_cand.sum())], tok.value, ms.value


def spec_verify_run_static(cfg: SvConfig, w_o_ptr: int, w_lm_ptr: int, inputs: SvInputs, outputs: SvOutputs,
                           stream: int | None = None) -> None:
    """The handle-free, allocation-free step of an fp32 model (see spec_verify.h)."""
    _check(lib().spec_verify_run_static(C.byref(cfg), C.c_void_p(w_o_ptr), C.c_void_p(w_lm_ptr), C.byref(inputs),
                                        C.byref(outputs), C.c_void_p(stream or 0)))


def spec_verify_destroy(h) -> None:
    _check(lib().spec_verify_destroy(h))


def spec_verify_profile(h, mode) -> None:
    """mode: 0/False off, 1/True every stage, 2 the LM-head stage only."""
    _check(lib().spec_verify_profile(h, int(mode)))


def spec_verify_stage_times(h) -> list[tuple[str, float]]:
    cap = 32
    names = (C.c_char_p * cap)()
    ms = (C.c_float * cap)()
    n = lib().spec_verify_stage_times(h, names, ms, cap)
    if n < 0:
        _check(n)
    return [(names[i].decode(), float(ms[i])) for i in range(min(n, cap))]


# ----------------------------------------------------------------------------
# torch convenience (marshalling of tensors into the C structs)
# ----------------------------------------------------------------------------


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def host_i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def host_i64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64))


class Verifier:
    """One handle: weights borrowed for its lifetime, outputs allocated with torch.

    `cfg` is an SvConfig; `w_o`, `w_lm` are contiguous device tensors."""

    def __init__(self, cfg: SvConfig, w_o, w_lm, prepared=None):
        import torch  # noqa: F401  (device memory)
        self.cfg = cfg
        self._w = (w_o, w_lm, prepared)
        if prepared is not None:
            # weights converted by spec_verify_prepare_weights, borrowed
            self.h = spec_verify_create_prepared(cfg, _ptr(prepared))
        else:
            self.h = spec_verify_create(cfg, _ptr(w_o), _ptr(w_lm))

    def close(self):
        if self.h is not None:
            spec_verify_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def alloc_outputs(self, n_rows: int, n_roots: int, device, with_logits: bool = False) -> dict:
        import torch
        i32 = dict(dtype=torch.int32, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        out = {"accept_len": torch.empty(n_roots, **i32), "bonus": torch.empty(n_roots, **i32),
               "last_row": torch.empty(n_roots, **i32), "surv_sum": torch.empty(n_roots, **f32),
               "argmax": torch.empty(n_rows, **i32), "row_max": torch.empty(n_rows, **f32),
               "row_lse": torch.empty(n_rows, **f32), "overlap": torch.empty(n_rows, **f32),
               "survival": torch.empty(n_rows, **f32)}
        out["logits"] = torch.empty(n_rows, self.cfg.vocab, **f32) if with_logits else None
        return out

    @staticmethod
    def make_structs(parent, pos, root_kv_off, root_kv_len, kv_k, kv_v, q_rows, k_rows, v_rows,
                     draft_ids, drafter_logits, outs: dict, mode: int = SV_MODE_GREEDY, u_accept=None,
                     u_bonus=None):
        """Build (SvInputs, SvOutputs, keepalive) from host arrays and device tensors."""
        parent, pos = host_i32(parent), host_i32(pos)
        root_kv_off, root_kv_len = host_i64(root_kv_off), host_i32(root_kv_len)
        n_rows = int(parent.shape[0])
        n_roots = int(root_kv_len.shape[0])
        kv_tokens = 0 if kv_k is None else int(kv_k.shape[0])
        inp = SvInputs(n_rows, n_roots,
                       parent.ctypes.data_as(C.POINTER(C.c_int32)), pos.ctypes.data_as(C.POINTER(C.c_int32)),
                       root_kv_off.ctypes.data_as(C.POINTER(C.c_int64)),
                       root_kv_len.ctypes.data_as(C.POINTER(C.c_int32)), kv_tokens,
                       _ptr(kv_k), _ptr(kv_v), _ptr(q_rows), _ptr(k_rows), _ptr(v_rows),
                       _ptr(draft_ids), _ptr(drafter_logits), int(mode), _ptr(u_accept), _ptr(u_bonus))
        o = SvOutputs(*[_ptr(outs.get(k)) for k, _ in SvOutputs._fields_])
        keep = (parent, pos, root_kv_off, root_kv_len)
        return inp, o, keep

    def run(self, inp: SvInputs, out: SvOutputs, stream: int | None = None):
        spec_verify_run(self.h, inp, out, stream)

    def commit(self, inp: SvInputs, out: SvOutputs, kv_k, kv_v, stream: int | None = None):
        spec_verify_commit(self.h, inp, out, _ptr(kv_k), _ptr(kv_v), stream)
