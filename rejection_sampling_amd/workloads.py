"""Seeded synthetic inputs for the verify step.

This module only draws random numbers and lays them out.  It holds none of the
verify arithmetic (no softmax, no filtering, no argmax, no sampling): the draft
distributions and the drafted tokens of each workload are built from these raw
pieces by whoever consumes them.  Tests and the smoke check build them with the
CPU oracle; the benchmark builds them with the library itself.

Every workload draws from ``numpy.random.Generator(PCG64(gen_seed))`` in the
fixed order written in each recipe, in fp32, and rounds logits to bf16 with
round-to-nearest-even on the bit pattern.  ``gen_seed = 1000*c + 1`` and the
Philox key ``seed = 1000*c + 7`` for workload c.  ``N(mu, s)`` means standard
deviation ``s``.

The five workloads stand in for the serving traffic the pages measure on
(speed tests over SPEED-Bench prompts and DS4 / DFLASH drafts); no dataset,
model or weights are involved.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

F32 = 0
BF16 = 1


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even.  Inputs are
    finite; NaN is not produced by any recipe."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact fp32 values."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Workload:
    """Raw random pieces of one verify step.

    ``rows_per_request`` gives the packed layout when it is fixed; the planner
    workload leaves it ``None`` and supplies ``confidence`` instead (its row
    total ``min(budget, R*block) + R`` is known without running the planner).
    """
    name: str
    num_requests: int
    vocab: int
    dtype: int
    logits: np.ndarray              # [rows, V] float32 (F32) or uint16 bf16 bits
    draft_logits: Optional[np.ndarray]  # same layout, or None (greedy-only)
    temperature: np.ndarray         # [R] float32
    top_k: np.ndarray               # [R] int32
    top_p: np.ndarray               # [R] float32
    request_id: np.ndarray          # [R] uint32
    position0: np.ndarray           # [R] uint32
    seed: int                       # Philox key
    rows_per_request: Optional[np.ndarray] = None  # [R] int32
    # greedy draft recipe (workload 1): which rows replace the argmax draft
    replace_mask: Optional[np.ndarray] = None      # [rows] bool
    replace_ids: Optional[np.ndarray] = None       # [rows] int32
    # planner recipe (workload 5)
    confidence: Optional[np.ndarray] = None        # [R, block] float32
    block: int = 0
    budget: int = 0

    @property
    def num_rows(self) -> int:
        return int(self.logits.shape[0])

    def qo_indptr(self) -> np.ndarray:
        assert self.rows_per_request is not None
        qo = np.zeros(self.num_requests + 1, dtype=np.int32)
        np.cumsum(self.rows_per_request, out=qo[1:])
        return qo

    def logits_f32(self) -> np.ndarray:
        return self.logits if self.dtype == F32 else bf16_to_f32(self.logits)


def _normal(g: np.random.Generator, shape, scale: float, loc: float = 0.0) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    if loc != 0.0:
        x += np.float32(loc)
    return x


def _common_ids(g: np.random.Generator, R: int):
    request_id = np.arange(R, dtype=np.uint32)
    position0 = g.integers(0, 4096, size=R).astype(np.uint32)
    return request_id, position0


def workload1(scale_rows: int = 1) -> Workload:
    """Greedy verify: 4 requests x (4 drafts + 1 bonus row), V 1024, fp32
    logits N(0, 2).  Drafts are the row argmax with ~30% replaced by uniform
    random ids (the replacement mask and ids are drawn here).
    Draw order: logits, replace mask, replace ids, position0."""
    c = 1
    g = np.random.Generator(np.random.PCG64(1000 * c + 1))
    R, gamma, V = 4 * scale_rows, 4, 1024
    rows = R * (gamma + 1)
    logits = _normal(g, (rows, V), 2.0)
    replace_mask = g.random(size=rows) < 0.3
    replace_ids = g.integers(0, V, size=rows).astype(np.int32)
    request_id, position0 = _common_ids(g, R)
    return Workload(
        name="greedy_4x5_v1024_f32", num_requests=R, vocab=V, dtype=F32,
        logits=logits, draft_logits=None,
        temperature=np.zeros(R, np.float32), top_k=np.zeros(R, np.int32),
        top_p=np.ones(R, np.float32), request_id=request_id, position0=position0,
        seed=1000 * c + 7, rows_per_request=np.full(R, gamma + 1, np.int32),
        replace_mask=replace_mask, replace_ids=replace_ids)


def _prob_workload(c: int, name: str, R: int, gamma: int, V: int, sigma: float,
                   peak: float, params) -> Workload:
    g = np.random.Generator(np.random.PCG64(1000 * c + 1))
    rows = R * (gamma + 1)
    logits = _normal(g, (rows, V), sigma)
    if peak:
        where = g.integers(0, V, size=rows)
        logits[np.arange(rows), where] += np.float32(peak)
    noise = _normal(g, (rows, V), 1.0)
    draft = logits + noise
    del noise
    T, k, P = params(g, R)
    request_id, position0 = _common_ids(g, R)
    return Workload(
        name=name, num_requests=R, vocab=V, dtype=BF16,
        logits=bf16_bits(logits), draft_logits=bf16_bits(draft),
        temperature=T, top_k=k, top_p=P, request_id=request_id, position0=position0,
        seed=1000 * c + 7, rows_per_request=np.full(R, gamma + 1, np.int32))


def workload2() -> Workload:
    """16 requests x (5 drafts + 1), V 32000, bf16 logits N(0,3), draft logits =
    target + N(0,1); T 0.7, top-k 50, top-p 0.9.
    Draw order: logits, draft noise, position0."""
    def params(g, R):
        return (np.full(R, 0.7, np.float32), np.full(R, 50, np.int32),
                np.full(R, 0.9, np.float32))
    return _prob_workload(2, "prob_16x6_v32000_bf16", 16, 5, 32000, 3.0, 0.0, params)


def workload3(num_requests: int = 128) -> Workload:
    """128 requests x 8-token blocks (7 drafts + 1 bonus = 1024 rows), V 248320,
    bf16 logits N(0,4) with +8 added at one seeded index per row; draft logits =
    target + N(0,1); T 1.0, top-k 20, top-p 0.95.
    Draw order: logits, peak indices, draft noise, position0."""
    def params(g, R):
        return (np.full(R, 1.0, np.float32), np.full(R, 20, np.int32),
                np.full(R, 0.95, np.float32))
    return _prob_workload(3, "prob_128x8_v248320_bf16", num_requests, 7, 248320, 4.0, 8.0,
                          params)


def workload4(num_requests: int = 512) -> Workload:
    """Mixed batch: 512 requests x 8-token blocks (4096 rows), V 129280, bf16
    logits N(0,3), draft = target + N(0,1).  A seeded permutation makes half the
    requests greedy (T 0); the rest draw T ~ U[0.3, 1.2], top-k from {0, 20, 50}
    and top-p from {1.0, 0.9}, uniformly.
    Draw order: logits, draft noise, permutation, T, k choice, P choice,
    position0."""
    def params(g, R):
        perm = g.permutation(R)
        greedy = np.zeros(R, bool)
        greedy[perm[: R // 2]] = True
        T = g.uniform(0.3, 1.2, size=R).astype(np.float32)
        k = np.array([0, 20, 50], np.int32)[g.integers(0, 3, size=R)]
        P = np.array([1.0, 0.9], np.float32)[g.integers(0, 2, size=R)]
        T[greedy] = 0.0
        return T, k, P
    return _prob_workload(4, "mixed_512x8_v129280_bf16", num_requests, 7, 129280, 3.0, 0.0,
                          params)


def workload5(num_requests: int = 256, budget: int = 1536) -> Workload:
    """Confidence-scheduled ragged verify: 256 requests, draft block 16.
    Confidence c[r, j] = sigmoid(z) * 0.95**j with z ~ N(1, 1.5).  The planner
    (global survival rank, budget 1536 drafted positions) packs
    min(budget, R*16) + R rows; they are generated here as one flat block, V
    248320, bf16 logits N(0,4) with a +8 planted index per row, draft = target +
    N(0,1); T 0.8, top-k off, top-p 0.95.
    Draw order: z, logits, peak indices, draft noise, position0."""
    c = 5
    g = np.random.Generator(np.random.PCG64(1000 * c + 1))
    R, B, V = num_requests, 16, 248320
    z = _normal(g, (R, B), 1.5, loc=1.0).astype(np.float64)
    decay = 0.95 ** np.arange(B, dtype=np.float64)
    conf = (1.0 / (1.0 + np.exp(-z)) * decay).astype(np.float32)
    rows = min(budget, R * B) + R
    logits = _normal(g, (rows, V), 4.0)
    where = g.integers(0, V, size=rows)
    logits[np.arange(rows), where] += np.float32(8.0)
    noise = _normal(g, (rows, V), 1.0)
    draft = logits + noise
    del noise
    request_id, position0 = _common_ids(g, R)
    return Workload(
        name="ragged_256xB16_v248320_bf16", num_requests=R, vocab=V, dtype=BF16,
        logits=bf16_bits(logits), draft_logits=bf16_bits(draft),
        temperature=np.full(R, 0.8, np.float32), top_k=np.zeros(R, np.int32),
        top_p=np.full(R, 0.95, np.float32), request_id=request_id, position0=position0,
        seed=1000 * c + 7, rows_per_request=None, confidence=conf, block=B, budget=budget)


def small_prob_workload(seed: int, R: int, gamma, V: int, sigma: float = 3.0,
                        noise: float = 1.0, T=0.8, k=0, P=1.0, dtype: int = BF16,
                        peak: float = 0.0) -> Workload:
    """A small probabilistic workload for parity cases.  ``gamma`` is an int or
    an array of per-request draft counts (ragged windows); T, k, P are scalars or
    [R] arrays.  Draw order: logits, peak indices (if any), draft noise,
    position0."""
    g = np.random.Generator(np.random.PCG64(seed))
    gam = np.broadcast_to(np.asarray(gamma, np.int32), (R,)).copy()
    rows = int((gam + 1).sum())
    logits = _normal(g, (rows, V), sigma)
    if peak:
        where = g.integers(0, V, size=rows)
        logits[np.arange(rows), where] += np.float32(peak)
    draft = logits + _normal(g, (rows, V), noise)
    request_id, position0 = _common_ids(g, R)
    T = np.broadcast_to(np.asarray(T, np.float32), (R,)).copy()
    k = np.broadcast_to(np.asarray(k, np.int32), (R,)).copy()
    P = np.broadcast_to(np.asarray(P, np.float32), (R,)).copy()
    if dtype == BF16:
        logits, draft = bf16_bits(logits), bf16_bits(draft)
    return Workload(
        name=f"small_{seed}", num_requests=R, vocab=V, dtype=dtype, logits=logits,
        draft_logits=draft, temperature=T, top_k=k, top_p=P, request_id=request_id,
        position0=position0, seed=seed * 7 + 3, rows_per_request=gam + 1)


WORKLOADS = {1: workload1, 2: workload2, 3: workload3, 4: workload4, 5: workload5}
