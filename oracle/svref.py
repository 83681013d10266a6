"""ctypes wrapper of the CPU oracle (oracle/libsvref.so).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg load this module.  It marshals numpy arrays to the oracle's C
functions and nothing else; the arithmetic lives in svref.cpp.

ctypes releases the GIL around each foreign call, so ``parallel_*`` helpers
run independent request ranges on a thread pool.  Each call is still the
single-threaded oracle; splitting by request does not change any result,
because every random draw is keyed by (seed, request id, position).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsvref.so")
SRC_PATH = os.path.join(HERE, "svref.cpp")

ROW_ACCEPT = 1
ROW_SAMPLED = 2
ROW_NEAR_RATIO = 4
ROW_NEAR_TOPP = 8
ROW_NEAR_RACE = 16
ROW_RESID_EMPTY = 32
ROW_BAD_DRAFT = 64

_lib = None


def build() -> str:
    """Compile the oracle with g++ (plain C++17, no fast-math, no contraction)."""
    cmd = ["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-Wall",
           "-shared", "-fPIC", "-o", LIB_PATH + ".tmp", SRC_PATH]
    subprocess.check_call(cmd)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


class Sampling(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_void_p), ("top_k", ctypes.c_void_p),
                ("top_p", ctypes.c_void_p), ("request_id", ctypes.c_void_p),
                ("position0", ctypes.c_void_p), ("seed", ctypes.c_uint64),
                ("flags", ctypes.c_uint32)]


def lib():
    """The loaded oracle.  SVREF_LIB names another build of svref.cpp (the
    mutation tests point it at deliberately broken copies)."""
    global _lib
    if _lib is None:
        path = os.environ.get("SVREF_LIB", LIB_PATH)
        if path == LIB_PATH and not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64, u32, u64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint64
        L.svref_philox4x32_10.argtypes = [P, P, P]
        L.svref_philox4x32_10.restype = None
        L.svref_uniform_accept.argtypes = [u64, u32, u32]
        L.svref_uniform_accept.restype = ctypes.c_double
        L.svref_uniform_race.argtypes = [u64, u32, u32, u32, u32]
        L.svref_uniform_race.restype = ctypes.c_double
        L.svref_build_target_probs.argtypes = [P, i32, i64, i32, i32, P, i32, P, P, i64, P, P, P,
                                               P, P, i32, P, P, P, P, P, P]
        L.svref_build_target_probs.restype = i32
        L.svref_rejection_sample.argtypes = [P, i32, i64, i32, P, i32, i32, P, P, i64, P, P, P, P,
                                             P, P, P, P, P, P]
        L.svref_rejection_sample.restype = i32
        L.svref_plan_windows.argtypes = [P, i64, i32, i32, i32, P, P, P]
        L.svref_plan_windows.restype = i32
        L.svref_accept_prefix.argtypes = [P, P, i32, P, P]
        L.svref_accept_prefix.restype = i32
        L.svref_acceptance_stats.argtypes = [P, P, i32, i32, P]
        L.svref_acceptance_stats.restype = i32
        L.svref_budget_from_costs.argtypes = [P, i64, i32, i32, P, i32, P, P]
        L.svref_budget_from_costs.restype = i32
        L.svref_est_init.argtypes = [P, i32]
        L.svref_est_init.restype = i32
        L.svref_est_feature.argtypes = [P, P, P, i32, P]
        L.svref_est_feature.restype = i32
        L.svref_est_predict.argtypes = [P, P, P, i32, P]
        L.svref_est_predict.restype = i32
        L.svref_est_observe.argtypes = [P, P, P, P, i32]
        L.svref_est_observe.restype = i32
        L.svref_sample_probs.argtypes = [P, i64, i32, i32, P, i32, P, P, u64, u32, P]
        L.svref_sample_probs.restype = i32
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def philox(key, ctr) -> np.ndarray:
    k = np.asarray(key, np.uint32)
    c = np.asarray(ctr, np.uint32)
    out = np.zeros(4, np.uint32)
    lib().svref_philox4x32_10(_p(k), _p(c), _p(out))
    return out


def uniform_accept(seed: int, rid: int, pos: int) -> float:
    return lib().svref_uniform_accept(seed, rid, pos)


def uniform_race(seed: int, rid: int, pos: int, tag: int, token: int) -> float:
    return lib().svref_uniform_race(seed, rid, pos, tag, token)


class _Params:
    """Keeps the per-request arrays alive while the C struct points at them."""

    def __init__(self, T, k, P, rid, pos0, seed, flags=0):
        self.T = _c(T, np.float32)
        self.k = _c(k, np.int32)
        self.P = _c(P, np.float32)
        self.rid = _c(rid, np.uint32)
        self.pos0 = _c(pos0, np.uint32)
        self.s = Sampling(_p(self.T), _p(self.k), _p(self.P), _p(self.rid), _p(self.pos0),
                          int(seed), int(flags))


BLOCK_VERIFY = 8


def _dt(logits):
    if logits.dtype == np.float32:
        return 0
    if logits.dtype == np.uint16:
        return 1
    raise TypeError("logits must be float32 or uint16 bf16 bits")


def build_target_probs(logits, qo, T, k=None, P=None, rid=None, pos0=None, seed=0,
                       want_probs=False, kmax=0):
    logits = np.ascontiguousarray(logits)
    rows, V = logits.shape
    R = len(qo) - 1
    qo = _c(qo, np.int32)
    prm = _Params(T, k, P, rid, pos0, seed)
    out = {
        "row_max": np.zeros(rows, np.float64),
        "row_argmax": np.zeros(rows, np.int32),
        "row_lse": np.zeros(rows, np.float64),
        "kept_count": np.zeros(rows, np.int32),
        "row_zn": np.zeros(rows, np.float64),
        "row_flags": np.zeros(rows, np.uint8),
        "row_zk": np.zeros(rows, np.float64),
        "kept_lo": np.zeros(rows, np.int32),
        "kept_hi": np.zeros(rows, np.int32),
    }
    kept_idx = np.zeros((rows, kmax), np.int32) if kmax > 0 else None
    order_idx = np.zeros((rows, kmax), np.int32) if kmax > 0 else None
    probs = np.zeros((rows, V), np.float64) if want_probs else None
    rc = lib().svref_build_target_probs(
        _p(logits), _dt(logits), V, rows, V, _p(qo), R, ctypes.byref(prm.s), _p(probs), V,
        _p(out["row_max"]), _p(out["row_argmax"]), _p(out["row_lse"]), _p(out["kept_count"]),
        _p(kept_idx), kmax, _p(out["row_zn"]), _p(out["row_flags"]), _p(out["row_zk"]),
        _p(out["kept_lo"]), _p(out["kept_hi"]), _p(order_idx))
    if rc != 0:
        raise ValueError(f"svref_build_target_probs returned {rc}")
    out["kept_idx"] = kept_idx
    out["order_idx"] = order_idx
    out["probs"] = probs
    return out


def rejection_sample(logits, qo, drafts, q, T, k=None, P=None, rid=None, pos0=None, seed=0,
                     verify_cap=None, block=False):
    """The verify step; block=True verifies sampled requests by block
    verification instead of the token-by-token ratio test."""
    logits = np.ascontiguousarray(logits)
    rows, V = logits.shape
    R = len(qo) - 1
    qo = _c(qo, np.int32)
    drafts = _c(drafts, np.int32)
    q = _c(q, np.float32)
    cap = _c(verify_cap, np.int32)
    prm = _Params(T, k, P, rid, pos0, seed, BLOCK_VERIFY if block else 0)
    out = {
        "accept_len": np.zeros(R, np.int32),
        "out_tokens": np.zeros(rows, np.int32),
        "next_token": np.zeros(R, np.int32),
        "row_flags": np.zeros(rows, np.uint8),
        "row_ratio": np.zeros(rows, np.float64),
        "row_u": np.zeros(rows, np.float64),
        "row_zk": np.zeros(rows, np.float64),
        "row_zn": np.zeros(rows, np.float64),
    }
    ldq = q.shape[1] if q is not None else V
    rc = lib().svref_rejection_sample(
        _p(logits), _dt(logits), V, V, _p(qo), R, rows, _p(drafts), _p(q), ldq, _p(cap),
        ctypes.byref(prm.s), _p(out["accept_len"]), _p(out["out_tokens"]),
        _p(out["next_token"]), _p(out["row_flags"]), _p(out["row_ratio"]), _p(out["row_u"]),
        _p(out["row_zk"]), _p(out["row_zn"]))
    if rc != 0:
        raise ValueError(f"svref_rejection_sample returned {rc}")
    return out


def plan_windows(conf, budget):
    conf = _c(conf, np.float32)
    R, B = conf.shape
    vl = np.zeros(R, np.int32)
    qo = np.zeros(R + 1, np.int32)
    surv = np.zeros((R, B), np.float32)
    rc = lib().svref_plan_windows(_p(conf), B, R, B, int(budget), _p(vl), _p(qo), _p(surv))
    if rc != 0:
        raise ValueError(f"svref_plan_windows returned {rc}")
    return vl, qo, surv


def budget_from_costs(conf, cost):
    """Verify budget maximising tau/cost over a step-cost table
    (svref_budget_from_costs): (budget, theta).  cost None: no table."""
    c = _c(conf, np.float32)
    R, B = (c.shape if c.ndim == 2 else (0, 0))
    tb = None if cost is None else _c(cost, np.float32)
    b = np.zeros(1, np.int32)
    th = np.zeros(1, np.float64)
    rc = lib().svref_budget_from_costs(_p(c), int(B), int(R), int(B),
                                       None if tb is None else _p(tb),
                                       0 if tb is None else int(tb.size), _p(b), _p(th))
    if rc != 0:
        raise ValueError(f"svref_budget_from_costs returned {rc}")
    return int(b[0]), float(th[0])


def acceptance_stats(accept_len, verify_len, block):
    """Acceptance and trim statistics (svref_acceptance_stats): int64 array
    [requests, trimmed, regret, sum accepted, sum window, offered[B], accepted[B]]."""
    L = _c(accept_len, np.int32)
    w = _c(verify_len, np.int32)
    out = np.zeros(5 + 2 * int(block), np.int64)
    rc = lib().svref_acceptance_stats(_p(L), _p(w), int(L.size), int(block), _p(out))
    if rc != 0:
        raise ValueError(f"svref_acceptance_stats returned {rc}")
    return out


EST_MAXB = 64
EST_REFIT = 100


class EstimatorState(ctypes.Structure):
    """Mirror of svref_estimator (oracle/svref.h)."""
    _fields_ = [("block", ctypes.c_int32), ("calls", ctypes.c_int32),
                ("refits", ctypes.c_int32), ("pad", ctypes.c_int32),
                ("slope", ctypes.c_double), ("bias", ctypes.c_double * EST_MAXB),
                ("h_ss", ctypes.c_double), ("g_s", ctypes.c_double), ("n_s", ctypes.c_double),
                ("h_sk", ctypes.c_double * EST_MAXB), ("h_kk", ctypes.c_double * EST_MAXB),
                ("g_k", ctypes.c_double * EST_MAXB), ("n_k", ctypes.c_double * EST_MAXB),
                ("last_ds", ctypes.c_double), ("last_db", ctypes.c_double * EST_MAXB)]


class Estimator:
    """The oracle's online acceptance estimator (svref_est_*)."""

    def __init__(self, block: int):
        self.st = EstimatorState()
        if lib().svref_est_init(ctypes.byref(self.st), int(block)) != 0:
            raise ValueError("bad block")
        self.block = int(block)

    @property
    def slope(self) -> float:
        return self.st.slope

    @property
    def bias(self) -> np.ndarray:
        return np.array(self.st.bias[: self.block])

    def predict(self, x, pos):
        x = _c(x, np.float64)
        pos = _c(pos, np.int32)
        out = np.zeros(x.size, np.float64)
        rc = lib().svref_est_predict(ctypes.byref(self.st), _p(x), _p(pos), int(x.size), _p(out))
        if rc != 0:
            raise ValueError(f"svref_est_predict returned {rc}")
        return out

    def observe(self, x, accept_len, verify_len):
        x = _c(x, np.float64)
        L = _c(accept_len, np.int32)
        w = _c(verify_len, np.int32)
        rc = lib().svref_est_observe(ctypes.byref(self.st), _p(x), _p(L), _p(w), int(L.size))
        if rc != 0:
            raise ValueError(f"svref_est_observe returned {rc}")


def est_feature(row_max, row_lse, t_eff):
    m = _c(row_max, np.float32)
    lse = _c(row_lse, np.float32)
    t = _c(t_eff, np.float32)
    out = np.zeros(m.size, np.float64)
    rc = lib().svref_est_feature(_p(m), _p(lse), _p(t), int(m.size), _p(out))
    if rc != 0:
        raise ValueError(f"svref_est_feature returned {rc}")
    return out


def accept_prefix(accepted, qo, verify_cap=None):
    acc = _c(accepted, np.uint8)
    qo = _c(qo, np.int32)
    cap = _c(verify_cap, np.int32)
    R = len(qo) - 1
    out = np.zeros(R, np.int32)
    rc = lib().svref_accept_prefix(_p(acc), _p(qo), R, _p(cap), _p(out))
    if rc != 0:
        raise ValueError(f"svref_accept_prefix returned {rc}")
    return out


def sample_probs(q, qo, rid, pos0, seed, tag=2):
    q = _c(q, np.float32)
    rows, V = q.shape
    qo = _c(qo, np.int32)
    rid = _c(rid, np.uint32)
    pos0 = _c(pos0, np.uint32)
    out = np.zeros(rows, np.int32)
    rc = lib().svref_sample_probs(_p(q), V, rows, V, _p(qo), len(qo) - 1, _p(rid), _p(pos0),
                                  int(seed), int(tag), _p(out))
    if rc != 0:
        raise ValueError(f"svref_sample_probs returned {rc}")
    return out


# ---------------------------------------------------------------------------
# request-sharded helpers (thread pool; each shard is one plain oracle call)
# ---------------------------------------------------------------------------

def _shards(qo, nshards):
    R = len(qo) - 1
    bounds = np.linspace(0, R, min(nshards, max(R, 1)) + 1).astype(int)
    return [(int(a), int(b)) for a, b in zip(bounds[:-1], bounds[1:]) if b > a]


def _sub(a, r0, r1):
    return None if a is None else np.asarray(a)[r0:r1]


def parallel_draft_probs(draft_logits, qo, T, k, P, rid, pos0, seed, threads=None):
    """Dense fp32 draft distributions q built by the oracle from draft logits
    with each request's own parameters (greedy requests give one-hot rows)."""
    threads = threads or min(16, os.cpu_count() or 1)
    rows, V = draft_logits.shape
    q = np.zeros((rows, V), np.float32)
    qo = np.asarray(qo, np.int32)

    def job(span):
        r0, r1 = span
        for a in range(r0, r1):  # one request per call bounds the fp64 temporary
            sa, sb = int(qo[a]), int(qo[a + 1])
            out = build_target_probs(draft_logits[sa:sb], qo[a:a + 2] - qo[a], _sub(T, a, a + 1),
                                     _sub(k, a, a + 1), _sub(P, a, a + 1), _sub(rid, a, a + 1),
                                     _sub(pos0, a, a + 1), seed, want_probs=True)
            q[sa:sb] = out["probs"].astype(np.float32)

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(job, _shards(qo, threads * 4)))
    return q


def parallel_argmax(logits, qo, threads=None):
    """Oracle argmax per row (greedy parameters)."""
    threads = threads or min(16, os.cpu_count() or 1)
    rows = logits.shape[0]
    qo = np.asarray(qo, np.int32)
    R = len(qo) - 1
    res = np.zeros(rows, np.int32)

    def job(span):
        r0, r1 = span
        s0, s1 = int(qo[r0]), int(qo[r1])
        out = build_target_probs(logits[s0:s1], qo[r0:r1 + 1] - qo[r0],
                                 np.zeros(r1 - r0, np.float32))
        res[s0:s1] = out["row_argmax"]

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(job, _shards(qo, threads * 4)))
    return res


def parallel_rejection_sample(logits, qo, drafts, q, T, k, P, rid, pos0, seed, verify_cap=None,
                              requests=None, threads=None, block=False):
    """Oracle verify over all requests, or over the listed ``requests`` only
    (each one as its own single-request call).  Returns per-request arrays and,
    for rows of covered requests, per-row arrays (rows of uncovered requests are
    left at -1 / 0)."""
    threads = threads or min(16, os.cpu_count() or 1)
    qo = np.asarray(qo, np.int32)
    R = len(qo) - 1
    rows = logits.shape[0]
    res = {
        "accept_len": np.full(R, -1, np.int32),
        "next_token": np.full(R, -1, np.int32),
        "out_tokens": np.full(rows, -1, np.int32),
        "row_flags": np.zeros(rows, np.uint8),
        "row_ratio": np.full(rows, np.nan),
        "row_u": np.full(rows, np.nan),
        "row_zk": np.full(rows, np.nan),
        "row_zn": np.full(rows, np.nan),
    }
    spans = _shards(qo, threads * 4) if requests is None else [(int(r), int(r) + 1)
                                                                for r in requests]

    def job(span):
        r0, r1 = span
        s0, s1 = int(qo[r0]), int(qo[r1])
        out = rejection_sample(logits[s0:s1], qo[r0:r1 + 1] - qo[r0], drafts[s0:s1],
                               None if q is None else q[s0:s1], _sub(T, r0, r1),
                               _sub(k, r0, r1), _sub(P, r0, r1), _sub(rid, r0, r1),
                               _sub(pos0, r0, r1), seed, _sub(verify_cap, r0, r1), block)
        res["accept_len"][r0:r1] = out["accept_len"]
        res["next_token"][r0:r1] = out["next_token"]
        for key in ("out_tokens", "row_flags", "row_ratio", "row_u", "row_zk", "row_zn"):
            res[key][s0:s1] = out[key]

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(job, spans))
    return res


def parallel_build(logits, qo, T, k, P, rid=None, pos0=None, seed=0, kmax=0, prob_rows=None,
                   threads=None):
    """Oracle target-distribution build over every request, sharded by request
    on a thread pool (each shard one plain call).  Per-row outputs for all
    rows; dense probabilities only for the rows listed in ``prob_rows`` (a
    dict row -> fp64 [V] array), which bounds the memory at large shapes."""
    threads = threads or min(16, os.cpu_count() or 1)
    qo = np.asarray(qo, np.int32)
    rows, V = logits.shape
    res = {
        "row_max": np.zeros(rows, np.float64), "row_argmax": np.zeros(rows, np.int32),
        "row_lse": np.zeros(rows, np.float64), "kept_count": np.zeros(rows, np.int32),
        "row_zn": np.zeros(rows, np.float64), "row_flags": np.zeros(rows, np.uint8),
        "row_zk": np.zeros(rows, np.float64), "kept_lo": np.zeros(rows, np.int32),
        "kept_hi": np.zeros(rows, np.int32),
        "kept_idx": np.zeros((rows, kmax), np.int32) if kmax else None,
        "order_idx": np.zeros((rows, kmax), np.int32) if kmax else None,
    }
    want = set() if prob_rows is None else set(int(i) for i in prob_rows)
    probs = {}

    def job(span):
        r0, r1 = span
        for a in range(r0, r1):
            sa, sb = int(qo[a]), int(qo[a + 1])
            if sb <= sa:
                continue
            dense = any(i in want for i in range(sa, sb))
            out = build_target_probs(logits[sa:sb], qo[a:a + 2] - qo[a], _sub(T, a, a + 1),
                                     _sub(k, a, a + 1), _sub(P, a, a + 1), _sub(rid, a, a + 1),
                                     _sub(pos0, a, a + 1), seed, want_probs=dense, kmax=kmax)
            for key in res:
                if res[key] is not None:
                    res[key][sa:sb] = out[key]
            if dense:
                for i in range(sa, sb):
                    if i in want:
                        probs[i] = out["probs"][i - sa].copy()

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(job, _shards(qo, threads * 4)))
    res["probs_rows"] = probs
    return res
