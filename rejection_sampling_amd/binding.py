"""Thin ctypes binding of libspecverify.so (include/spec_verify.h).

Argument marshalling only: torch tensors are checked for device, dtype and
layout and passed as raw pointers with the current HIP stream.  Every step of
the verify path runs in the library's HIP kernels; there is no host or torch
fallback.  Importing this module on a machine without the built library, or
calling it without a GPU, raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libspecverify.so")

SV_F32, SV_BF16 = 0, 1
SV_ALL_GREEDY = 1
SV_CHECK = 2
SV_LIST_BOUNDED = 4
SV_BLOCK_VERIFY = 8
LAYOUT_START, LAYOUT_ORDER, LAYOUT_END = 1, 2, 4
LIST_CAP = 4096  # kept-set entries a row can list (top-k bound of SV_LIST_BOUNDED)
TOPK_SINGLE_PASS = 256  # largest top-k the streaming pass selects by itself
BUDGET_ONE_GROUP = 4096  # drafted positions plan_budget sorts in one workgroup (no workspace)
BUDGET_MAX = 1 << 20     # drafted positions plan_budget accepts
ROW_ACCEPT, ROW_SAMPLED, ROW_RESID_EMPTY = 1, 2, 32
KERNEL_IDS = {"row_pass": 0, "finalize": 1, "build_out": 2, "planner": 3, "accept_prefix": 4,
              "race_segment": 5, "race_finish": 6, "acceptance_stats": 7, "check_layout": 8,
              "diagnostics": 9}

EXPORTS = [
    "spec_verify_workspace_bytes", "spec_verify_build_target_probs",
    "spec_verify_rejection_sample", "spec_verify_plan_windows", "spec_verify_accept_prefix",
    "spec_verify_status_string", "spec_verify_last_error", "spec_verify_profile_enable",
    "spec_verify_profile_read", "spec_verify_profile_reset", "spec_verify_acceptance_stats",
    "spec_verify_estimator_state_doubles", "spec_verify_estimator_init",
    "spec_verify_estimator_predict", "spec_verify_estimator_observe", "spec_verify_plan_budget",
    "spec_verify_check_layout", "spec_verify_row_diagnostics",
    "spec_verify_rejection_sample_noalloc",
]


class Sampling(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_void_p), ("top_k", ctypes.c_void_p),
                ("top_p", ctypes.c_void_p), ("request_id", ctypes.c_void_p),
                ("position0", ctypes.c_void_p), ("seed", ctypes.c_uint64),
                ("flags", ctypes.c_uint32), ("row_order", ctypes.c_void_p)]


_lib = None


def load(path: str = LIB_PATH):
    """Load the library (no GPU needed to load it)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m rejection_sampling_amd.build` "
                           "or __graft_entry__.build()")
    L = ctypes.CDLL(path)
    P, i32, i64, u64, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                            ctypes.c_size_t)
    L.spec_verify_workspace_bytes.argtypes = [i32, i32, i32, i32]
    L.spec_verify_workspace_bytes.restype = sz
    L.spec_verify_build_target_probs.argtypes = [P, i32, i64, i32, i32, P, i32, P, P, i64, P, P,
                                                 P, P, P, i32, P, sz, P]
    L.spec_verify_build_target_probs.restype = i32
    L.spec_verify_rejection_sample.argtypes = [P, i32, i64, i32, P, i32, i32, P, P, i64, P, P, P,
                                               P, P, P, P, sz, P]
    L.spec_verify_rejection_sample.restype = i32
    L.spec_verify_rejection_sample_noalloc.argtypes = [P, i32, i64, i32, P, i32, i32, P, P, i64,
                                                       P, P, P, P, P, P, P]
    L.spec_verify_rejection_sample_noalloc.restype = i32
    L.spec_verify_plan_windows.argtypes = [P, i64, i32, i32, i32, P, P, P, P, sz, P]
    L.spec_verify_plan_windows.restype = i32
    L.spec_verify_plan_budget.argtypes = [P, i64, i32, i32, P, i32, P, P, P, sz, P]
    L.spec_verify_plan_budget.restype = i32
    L.spec_verify_check_layout.argtypes = [P, i32, i32, P, P]
    L.spec_verify_check_layout.restype = i32
    L.spec_verify_row_diagnostics.argtypes = [P, sz, i32, P, P, P, P, P]
    L.spec_verify_row_diagnostics.restype = i32
    L.spec_verify_accept_prefix.argtypes = [P, P, i32, P, P, P]
    L.spec_verify_accept_prefix.restype = i32
    L.spec_verify_acceptance_stats.argtypes = [P, P, i32, i32, P, P]
    L.spec_verify_acceptance_stats.restype = i32
    L.spec_verify_estimator_state_doubles.argtypes = [i32]
    L.spec_verify_estimator_state_doubles.restype = sz
    L.spec_verify_estimator_init.argtypes = [P, i32, P]
    L.spec_verify_estimator_init.restype = i32
    L.spec_verify_estimator_predict.argtypes = [P, P, P, i32, i32, P, P, P, P]
    L.spec_verify_estimator_predict.restype = i32
    L.spec_verify_estimator_observe.argtypes = [P, P, P, i32, i32, P, P]
    L.spec_verify_estimator_observe.restype = i32
    L.spec_verify_status_string.argtypes = [i32]
    L.spec_verify_status_string.restype = ctypes.c_char_p
    L.spec_verify_last_error.argtypes = []
    L.spec_verify_last_error.restype = ctypes.c_char_p
    L.spec_verify_profile_enable.argtypes = [i32]
    L.spec_verify_profile_enable.restype = i32
    L.spec_verify_profile_read.argtypes = [i32, P, P]
    L.spec_verify_profile_read.restype = i32
    L.spec_verify_profile_reset.argtypes = []
    L.spec_verify_profile_reset.restype = i32
    _lib = L
    return L


class SpecVerifyError(RuntimeError):
    pass


def _check(rc: int):
    if rc != 0:
        L = load()
        raise SpecVerifyError(f"{L.spec_verify_status_string(rc).decode()} ({rc}): "
                              f"{L.spec_verify_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dev(t: Optional[torch.Tensor], dtype, name):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _logits(t: torch.Tensor, name="logits"):
    if not t.is_cuda or t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D device tensor with unit column stride")
    if t.dtype == torch.bfloat16:
        return SV_BF16
    if t.dtype == torch.float32:
        return SV_F32
    raise ValueError(f"{name} must be bfloat16 or float32")


def _stream():
    return torch.cuda.current_stream().cuda_stream


_ws_cache = {}


def _device(device=None) -> torch.device:
    """A device with its index filled in (the workspace cache key)."""
    dev = torch.device(device or "cuda")
    if dev.index is None:
        dev = torch.device(dev.type, torch.cuda.current_device())
    return dev


def workspace(num_rows: int, vocab: int, num_requests: int, block: int = 0,
              device=None) -> torch.Tensor:
    """A cached device workspace of at least the queried size."""
    n = int(load().spec_verify_workspace_bytes(num_rows, vocab, num_requests, block))
    dev = _device(device)
    cur = _ws_cache.get(dev)
    if cur is None or cur.numel() < n:
        cur = torch.empty(max(n, 1 << 20), dtype=torch.uint8, device=dev)
        _ws_cache[dev] = cur
    return cur


class Params:
    """Per-request sampling values as device tensors (kept alive with the
    call).  Nothing here reads device memory: the flags are the caller's
    (all_greedy, list_bounded: hints the caller knows from its own host-side
    request parameters; check: the device-side layout check of SV_CHECK).
    Params.from_host() takes host arrays instead, derives the hints from them
    and uploads the values once."""

    def __init__(self, temperature, top_k=None, top_p=None, request_id=None, position0=None,
                 seed: int = 0, all_greedy: bool = False, list_bounded: bool = False,
                 check: bool = False, block: bool = False):
        self.T = _dev(temperature, torch.float32, "temperature")
        self.k = _dev(top_k, torch.int32, "top_k")
        self.P = _dev(top_p, torch.float32, "top_p")
        # request ids and positions are uint32 in the ABI; int32 tensors carry
        # the same bits
        self.rid = _dev(request_id, torch.int32, "request_id")
        self.pos0 = _dev(position0, torch.int32, "position0")
        self.host = None   # (T, k, P) host arrays when built by from_host
        flags = ((SV_ALL_GREEDY if all_greedy else 0) | (SV_LIST_BOUNDED if list_bounded else 0) |
                 (SV_CHECK if check else 0) | (SV_BLOCK_VERIFY if block else 0))
        self.s = Sampling(_ptr(self.T), _ptr(self.k), _ptr(self.P), _ptr(self.rid),
                          _ptr(self.pos0), int(seed) & ((1 << 64) - 1), flags, None)

    @classmethod
    def from_host(cls, temperature, top_k=None, top_p=None, request_id=None, position0=None,
                  seed: int = 0, device="cuda", check: bool = False, block: bool = False):
        """Build from host (numpy or CPU) arrays: every request greedy sets
        SV_ALL_GREEDY, every sampled request with 0 < top_k <= 4096 sets
        SV_LIST_BOUNDED.  The arrays are uploaded once, here."""
        import numpy as np
        T = np.ascontiguousarray(np.asarray(temperature, np.float32))
        R = T.size
        k = None if top_k is None else np.ascontiguousarray(np.asarray(top_k, np.int32))
        P = None if top_p is None else np.ascontiguousarray(np.asarray(top_p, np.float32))
        kk = np.zeros(R, np.int32) if k is None else k
        all_greedy, list_bounded = sampling_hints(T, kk)
        def up(a, dt):
            return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dt)).to(device)

        def u32(a):  # uint32 values travel as int32 tensors with the same bits
            return None if a is None else torch.from_numpy(
                np.ascontiguousarray(a, np.uint32).view(np.int32)).to(device)
        prm = cls(up(T, np.float32), up(k, np.int32), up(P, np.float32), u32(request_id),
                  u32(position0), seed, all_greedy, list_bounded, check, block)
        prm.host = (T, kk, np.ones(R, np.float32) if P is None else P)
        return prm


def sampling_hints(temperature, top_k):
    """(all_greedy, list_bounded) from host values: no request samples (T > 0),
    and every sampled request has 0 < top_k <= LIST_CAP."""
    import numpy as np
    T = np.asarray(temperature, np.float32)
    k = np.asarray(top_k, np.int32)
    sampled = T > 0
    return (not bool(sampled.any()),
            bool(((k[sampled] > 0) & (k[sampled] <= LIST_CAP)).all()))


def heavy_first_order(qo_indptr, params: Params, vocab: int, device="cuda"):
    """Row schedule (a device int32 permutation) with the rows of requests that
    may take the multi-pass exact path first: sampled, top-k off with top-p
    on, or top-k above the single-pass limit.  Computed on the host from the
    host qo_indptr and the host values Params.from_host kept; None when no
    reordering helps (no heavy request, or only heavy ones)."""
    import numpy as np
    if params.host is None:
        raise ValueError("heavy_first_order needs Params.from_host (host sampling values)")
    Th, kh, Ph = params.host
    k_off = (kh <= 0) | (kh >= vocab)
    heavy = (Th > 0) & ((k_off & (Ph < 1) & (Ph > 0)) | ((kh > TOPK_SINGLE_PASS) & ~k_off))
    if not heavy.any() or heavy.all():
        return None
    qo = np.asarray(qo_indptr, np.int64)
    rows = np.arange(int(qo[-1]), dtype=np.int64)
    req = np.searchsorted(qo[1:], rows, side="right")
    first = heavy[req]
    order = np.concatenate([rows[first], rows[~first]]).astype(np.int32)
    return torch.from_numpy(order).to(device)


def build_target_probs(logits: torch.Tensor, qo_indptr: torch.Tensor, params: Params,
                       want_probs: bool = False, kmax: int = 0):
    dt = _logits(logits)
    rows, V = logits.shape
    qo = _dev(qo_indptr, torch.int32, "qo_indptr")
    R = qo.numel() - 1
    dev = logits.device
    out = {
        "row_max": torch.empty(rows, dtype=torch.float32, device=dev),
        "row_argmax": torch.empty(rows, dtype=torch.int32, device=dev),
        "row_lse": torch.empty(rows, dtype=torch.float32, device=dev),
        "kept_count": torch.empty(rows, dtype=torch.int32, device=dev),
        "kept_idx": torch.empty((rows, kmax), dtype=torch.int32, device=dev) if kmax else None,
        "probs": torch.empty((rows, V), dtype=torch.float32, device=dev) if want_probs else None,
    }
    ws = workspace(rows, V, R, 0, dev)
    rc = load().spec_verify_build_target_probs(
        _ptr(logits), dt, logits.stride(0), rows, V, _ptr(qo), R, ctypes.byref(params.s),
        _ptr(out["probs"]), V, _ptr(out["row_max"]), _ptr(out["row_argmax"]),
        _ptr(out["row_lse"]), _ptr(out["kept_count"]), _ptr(out["kept_idx"]), kmax, _ptr(ws),
        ws.numel(), _stream())
    _check(rc)
    return out


def rejection_sample(logits: torch.Tensor, qo_indptr: torch.Tensor, draft_tokens: torch.Tensor,
                     draft_probs: Optional[torch.Tensor], params: Params,
                     verify_cap: Optional[torch.Tensor] = None, out=None):
    dt = _logits(logits)
    rows, V = logits.shape
    qo = _dev(qo_indptr, torch.int32, "qo_indptr")
    R = qo.numel() - 1
    dev = logits.device
    d = _dev(draft_tokens, torch.int32, "draft_tokens")
    if draft_probs is not None:
        if draft_probs.dtype != torch.float32 or not draft_probs.is_cuda or \
                draft_probs.stride(1) != 1:
            raise ValueError("draft_probs must be a 2-D fp32 device tensor")
    cap = _dev(verify_cap, torch.int32, "verify_cap")
    if out is None:
        out = {
            "accept_len": torch.empty(R, dtype=torch.int32, device=dev),
            "out_tokens": torch.empty(rows, dtype=torch.int32, device=dev),
            "next_token": torch.empty(R, dtype=torch.int32, device=dev),
            "row_flags": torch.empty(rows, dtype=torch.uint8, device=dev),
        }
    ws = workspace(rows, V, R, 0, dev)
    ldq = draft_probs.stride(0) if draft_probs is not None else V
    rc = load().spec_verify_rejection_sample(
        _ptr(logits), dt, logits.stride(0), V, _ptr(qo), R, rows, _ptr(d), _ptr(draft_probs), ldq,
        _ptr(cap), ctypes.byref(params.s), _ptr(out["accept_len"]), _ptr(out["out_tokens"]),
        _ptr(out["next_token"]), _ptr(out["row_flags"]), _ptr(ws), ws.numel(), _stream())
    _check(rc)
    return out


NOALLOC_MAX_ROWS = NOALLOC_MAX_REQUESTS = 1024


def rejection_sample_noalloc(logits: torch.Tensor, qo_indptr: torch.Tensor,
                             draft_tokens: torch.Tensor, draft_probs: Optional[torch.Tensor],
                             params: Params, out, verify_cap: Optional[torch.Tensor] = None):
    """spec_verify_rejection_sample_noalloc: the verify step with the
    library's static per-device scratch instead of a workspace.  `out` holds
    the caller's output tensors (accept_len, out_tokens, next_token,
    row_flags), so neither the call nor this wrapper allocates."""
    dt = _logits(logits)
    rows, V = logits.shape
    qo = _dev(qo_indptr, torch.int32, "qo_indptr")
    R = qo.numel() - 1
    d = _dev(draft_tokens, torch.int32, "draft_tokens")
    if draft_probs is not None and (draft_probs.dtype != torch.float32 or
                                    not draft_probs.is_cuda or draft_probs.stride(1) != 1):
        raise ValueError("draft_probs must be a 2-D fp32 device tensor")
    cap = _dev(verify_cap, torch.int32, "verify_cap")
    ldq = draft_probs.stride(0) if draft_probs is not None else V
    rc = load().spec_verify_rejection_sample_noalloc(
        _ptr(logits), dt, logits.stride(0), V, _ptr(qo), R, rows, _ptr(d), _ptr(draft_probs), ldq,
        _ptr(cap), ctypes.byref(params.s), _ptr(out["accept_len"]), _ptr(out["out_tokens"]),
        _ptr(out["next_token"]), _ptr(out.get("row_flags")), _stream())
    _check(rc)
    return out


class PreparedRejectionSample:
    """rejection_sample with its arguments checked and marshalled once: each
    call is one foreign call on the stream current at construction.  The
    tensors must stay alive and keep their shapes and storage.  row_order
    (device int32 [rows], e.g. from heavy_first_order) schedules the rows."""

    def __init__(self, logits, qo_indptr, draft_tokens, draft_probs, params: Params,
                 verify_cap=None, out=None, row_order: Optional[torch.Tensor] = None):
        dt = _logits(logits)
        rows, V = logits.shape
        qo = _dev(qo_indptr, torch.int32, "qo_indptr")
        R = qo.numel() - 1
        d = _dev(draft_tokens, torch.int32, "draft_tokens")
        if draft_probs is not None and (draft_probs.dtype != torch.float32 or
                                        not draft_probs.is_cuda or draft_probs.stride(1) != 1):
            raise ValueError("draft_probs must be a 2-D fp32 device tensor")
        cap = _dev(verify_cap, torch.int32, "verify_cap")
        dev = logits.device
        if out is None:
            out = {
                "accept_len": torch.empty(R, dtype=torch.int32, device=dev),
                "out_tokens": torch.empty(rows, dtype=torch.int32, device=dev),
                "next_token": torch.empty(R, dtype=torch.int32, device=dev),
                "row_flags": torch.empty(rows, dtype=torch.uint8, device=dev),
            }
        ws = workspace(rows, V, R, 0, dev)
        ldq = draft_probs.stride(0) if draft_probs is not None else V
        # this call's copy of the sampling block, with the caller's row order
        order = _dev(row_order, torch.int32, "row_order")
        if order is not None and order.numel() != rows:
            raise ValueError("row_order must hold one entry per row")
        self._s = Sampling(*[getattr(params.s, f) for f, _ in Sampling._fields_])
        self._s.row_order = _ptr(order)
        self.out = out
        self._keep = (logits, qo, d, draft_probs, cap, params, ws, order)
        self._fn = load().spec_verify_rejection_sample
        self._args = (_ptr(logits), dt, logits.stride(0), V, _ptr(qo), R, rows, _ptr(d),
                      _ptr(draft_probs), ldq, _ptr(cap), ctypes.byref(self._s),
                      _ptr(out["accept_len"]), _ptr(out["out_tokens"]), _ptr(out["next_token"]),
                      _ptr(out["row_flags"]), _ptr(ws), ws.numel(), _stream())

    def __call__(self):
        rc = self._fn(*self._args)
        if rc:
            _check(rc)
        return self.out


def plan_windows(confidence: torch.Tensor, budget: int, want_survival: bool = True):
    conf = _dev(confidence, torch.float32, "confidence")
    R, B = conf.shape
    dev = conf.device
    vl = torch.empty(R, dtype=torch.int32, device=dev)
    qo = torch.empty(R + 1, dtype=torch.int32, device=dev)
    surv = torch.empty((R, B), dtype=torch.float32, device=dev) if want_survival else None
    ws = workspace(0, 1, R, B, dev)
    rc = load().spec_verify_plan_windows(_ptr(conf), B, R, B, int(budget), _ptr(vl), _ptr(qo),
                                         _ptr(surv), _ptr(ws), ws.numel(), _stream())
    _check(rc)
    return vl, qo, surv


def plan_budget(confidence: torch.Tensor, cost: Optional[torch.Tensor]):
    """Verify budget maximising tau/cost over a step-cost table
    (spec_verify_plan_budget): (budget int32 [1], theta fp64 [1]), both on the
    device.  cost None: no table (no trim)."""
    conf = _dev(confidence, torch.float32, "confidence")
    R, B = conf.shape
    tb = _dev(cost, torch.float32, "cost")
    budget = torch.empty(1, dtype=torch.int32, device=conf.device)
    theta = torch.empty(1, dtype=torch.float64, device=conf.device)
    ws = workspace(0, 1, R, B, conf.device) if R * B > BUDGET_ONE_GROUP else None
    rc = load().spec_verify_plan_budget(_ptr(conf), B, R, B, _ptr(tb),
                                        0 if tb is None else tb.numel(), _ptr(budget),
                                        _ptr(theta), _ptr(ws), 0 if ws is None else ws.numel(),
                                        _stream())
    _check(rc)
    return budget, theta


def check_layout(qo_indptr: torch.Tensor, num_rows: int) -> torch.Tensor:
    """Device int32 [1]: 0, or the LAYOUT_* bits qo_indptr violates
    (spec_verify_check_layout)."""
    qo = _dev(qo_indptr, torch.int32, "qo_indptr")
    word = torch.empty(1, dtype=torch.int32, device=qo.device)
    _check(load().spec_verify_check_layout(_ptr(qo), qo.numel() - 1, int(num_rows), _ptr(word),
                                           _stream()))
    return word


def row_diagnostics(num_rows: int, ws: Optional[torch.Tensor] = None, device=None):
    """Per-row Z_K, Z_N, p(d) and mode recorded by the last call on the
    workspace `ws` (default: this module's cached workspace of the device)."""
    dev = _device(device)
    ws = _ws_cache.get(dev) if ws is None else ws
    if ws is None:
        raise ValueError("no workspace: run a verify or build call first")
    out = {"zk": torch.empty(num_rows, dtype=torch.float64, device=dev),
           "zn": torch.empty(num_rows, dtype=torch.float64, device=dev),
           "pd": torch.empty(num_rows, dtype=torch.float64, device=dev),
           "mode": torch.empty(num_rows, dtype=torch.int32, device=dev)}
    _check(load().spec_verify_row_diagnostics(_ptr(ws), ws.numel(), int(num_rows),
                                              _ptr(out["zk"]), _ptr(out["zn"]), _ptr(out["pd"]),
                                              _ptr(out["mode"]), _stream()))
    return out


def workspace_check_word(ws: Optional[torch.Tensor] = None, device=None) -> torch.Tensor:
    """The SV_CHECK layout word of the last call on `ws` (a device view)."""
    ws = _ws_cache.get(_device(device)) if ws is None else ws
    if ws is None:
        raise ValueError("no workspace: run a verify or build call first")
    return ws[:4].view(torch.int32)


def accept_prefix(accepted: torch.Tensor, qo_indptr: torch.Tensor,
                  verify_cap: Optional[torch.Tensor] = None):
    acc = _dev(accepted, torch.uint8, "accepted")
    qo = _dev(qo_indptr, torch.int32, "qo_indptr")
    cap = _dev(verify_cap, torch.int32, "verify_cap")
    R = qo.numel() - 1
    out = torch.empty(R, dtype=torch.int32, device=qo.device)
    rc = load().spec_verify_accept_prefix(_ptr(acc), _ptr(qo), R, _ptr(cap), _ptr(out), _stream())
    _check(rc)
    return out


def acceptance_stats(accept_len: torch.Tensor, verify_len: torch.Tensor, block: int):
    """Acceptance and trim statistics of one verify step: an int64 device
    tensor [requests, trimmed, regret, sum accepted, sum window, offered[B],
    accepted[B]] (spec_verify_acceptance_stats)."""
    L = _dev(accept_len, torch.int32, "accept_len")
    w = _dev(verify_len, torch.int32, "verify_len")
    if L.numel() != w.numel():
        raise ValueError("accept_len and verify_len differ in length")
    out = torch.empty(5 + 2 * int(block), dtype=torch.int64, device=L.device)
    rc = load().spec_verify_acceptance_stats(_ptr(L), _ptr(w), L.numel(), int(block), _ptr(out),
                                             _stream())
    _check(rc)
    return out


class AcceptanceEstimator:
    """The online acceptance estimator on the device: a state tensor of
    doubles, initialised on construction; predict() gives the planner's
    confidences from the draft build's row max and lse, observe() feeds a
    verified step back (spec_verify_estimator_*)."""

    def __init__(self, block: int, device=None):
        self.block = int(block)
        n = int(load().spec_verify_estimator_state_doubles(self.block))
        if n == 0:
            raise ValueError("block must be in [1, 64]")
        self.state = torch.empty(n, dtype=torch.float64, device=device or "cuda")
        _check(load().spec_verify_estimator_init(_ptr(self.state), self.block, _stream()))

    def predict(self, row_max: torch.Tensor, row_lse: torch.Tensor,
                temperature: Optional[torch.Tensor] = None):
        m = _dev(row_max, torch.float32, "row_max")
        lse = _dev(row_lse, torch.float32, "row_lse")
        T = _dev(temperature, torch.float32, "temperature")
        if m.numel() % self.block or lse.numel() != m.numel():
            raise ValueError("row_max / row_lse must hold num_requests * block rows")
        R = m.numel() // self.block
        feat = torch.empty((R, self.block), dtype=torch.float64, device=m.device)
        conf = torch.empty((R, self.block), dtype=torch.float32, device=m.device)
        _check(load().spec_verify_estimator_predict(_ptr(m), _ptr(lse), _ptr(T), R, self.block,
                                                    _ptr(self.state), _ptr(feat), _ptr(conf),
                                                    _stream()))
        return feat, conf

    def observe(self, feature: torch.Tensor, accept_len: torch.Tensor, verify_len: torch.Tensor):
        f = _dev(feature, torch.float64, "feature")
        L = _dev(accept_len, torch.int32, "accept_len")
        w = _dev(verify_len, torch.int32, "verify_len")
        if L.numel() != w.numel() or f.numel() != L.numel() * self.block:
            raise ValueError("feature must be [num_requests, block]")
        _check(load().spec_verify_estimator_observe(_ptr(f), _ptr(L), _ptr(w), L.numel(),
                                                    self.block, _ptr(self.state), _stream()))

    def coefficients(self):
        """(slope, intercepts, refits) read back to the host (synchronizes)."""
        st = self.state.cpu().numpy()
        B = self.block
        return float(st[0]), st[1:1 + B].copy(), int(st[5 + 5 * B])


def profile_enable(on: bool = True):
    _check(load().spec_verify_profile_enable(1 if on else 0))


def profile_reset():
    _check(load().spec_verify_profile_reset())


def profile_read(kernel: str):
    n = ctypes.c_int64(0)
    ms = ctypes.c_double(0.0)
    _check(load().spec_verify_profile_read(KERNEL_IDS[kernel], ctypes.byref(n), ctypes.byref(ms)))
    return int(n.value), float(ms.value)
