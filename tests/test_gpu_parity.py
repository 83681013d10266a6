"""GPU parity of the verify step against the CPU oracle (through the C ABI).

Every case compares every request and row with the oracle, the five
workloads at their full sizes included (the oracle runs sharded by request
over host threads; each shard is the plain single-threaded oracle, and
results are keyed by request id and position, so sharding changes nothing).
Tolerances: integers bit-exact; probabilities 1e-5 relative; lse 1e-4
absolute; decision mismatches only on oracle-flagged near ties, at most 1e-4
of the rows.  On the workloads the GPU's own decision quantities (Z_K and the
ratio) are also checked against the oracle's to half the near-tie bands.
"""
import os

import numpy as np
import pytest
import torch

from oracle import svref
from rejection_sampling_amd import workloads as W
from tests.gpu_common import (compare_build, compare_margins, compare_verify, dev_f32, dev_i32,
                              dev_logits, gpu_verify, make_drafts, oracle_verify, params_for,
                              progress)

pytestmark = pytest.mark.gpu

THREADS = min(16, os.cpu_count() or 1)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from rejection_sampling_amd import binding
    binding.load()   # fails loudly when the library is missing
    yield


# ------------------------------------------------------------ small cases
GRID = [
    # (T, k, P)
    (0.0, 0, 1.0), (0.8, 0, 1.0), (0.8, 0, 0.9), (1.0, 20, 0.95), (0.7, 50, 0.9),
    (1.3, 5, 1.0), (0.5, 1, 0.5), (1.0, 2000, 0.9), (1.1, 3000, 1.0), (0.9, 0, 0.0),
    (1.2, 1024, 0.97), (0.6, 0, 0.5),
]


def _small(seed, V, dtype=W.BF16, R=24, sigma=3.0, peak=0.0):
    g = np.random.default_rng(seed)
    gam = g.integers(0, 8, size=R)
    choice = g.integers(0, len(GRID), size=R)
    T = np.array([GRID[c][0] for c in choice], np.float32)
    k = np.array([GRID[c][1] for c in choice], np.int32)
    P = np.array([GRID[c][2] for c in choice], np.float32)
    return W.small_prob_workload(seed, R, gam, V, sigma=sigma, T=T, k=k, P=P, dtype=dtype,
                                 peak=peak)


def _run_small(w, verify_cap=None, label=""):
    qo = w.qo_indptr()
    q, d = make_drafts(w, qo, THREADS)
    progress(f"{label}: rows={w.num_rows} V={w.vocab} dtype={w.dtype}")
    gpu = gpu_verify(w, qo, d, q, verify_cap)
    ref = oracle_verify(w, qo, d, q, verify_cap, threads=THREADS)
    compare_verify(gpu, ref, qo, cap=verify_cap, label=label)
    # structural properties
    for r in range(w.num_requests):
        s, e = qo[r], qo[r + 1]
        L = gpu["accept_len"][r]
        assert 0 <= L <= e - s - 1
        assert gpu["out_tokens"][s + L] == gpu["next_token"][r]
        assert np.all(gpu["out_tokens"][s + L + 1:e] == -1)
        assert 0 <= gpu["next_token"][r] < w.vocab
    return gpu, ref


@pytest.mark.parametrize("V", [20007, 32000, 4099])
def test_small_grid_bf16(V):
    _run_small(_small(11 + V, V), label=f"bf16 grid V={V}")


def test_small_grid_fp32():
    _run_small(_small(5, 9001, dtype=W.F32), label="fp32 grid")


def test_small_grid_peaked_bf16():
    _run_small(_small(6, 50000, sigma=4.0, peak=8.0), label="peaked bf16 grid")


def test_split_race_and_one_workgroup_race():
    """Rows sampled over the whole vocabulary (top-k off): split over
    workgroups by default, and raced by one workgroup each when the
    bounded-list hint is given although it does not hold.  Both match the
    oracle."""
    w = _small(12, 40000, R=24)
    qo = w.qo_indptr()
    q, d = make_drafts(w, qo, THREADS)
    ref = oracle_verify(w, qo, d, q, threads=THREADS)
    assert np.any((w.top_k == 0) & (w.temperature > 0))
    for bounded in (False, True):
        progress(f"race split, list_bounded={bounded}")
        gpu = gpu_verify(w, qo, d, q, list_bounded=bounded)
        compare_verify(gpu, ref, qo, label=f"list_bounded={bounded}")


def test_zero_residual_race_falls_back_to_p():
    """Draft probabilities at twice the target's on every token (q is then no
    distribution, which neither side needs): every rejection leaves a residual
    that is zero on the whole kept set, so the emitted token is raced over p.
    Whole-vocabulary kept sets (top-k off; top-p off, or 0.999 on flat rows
    for kept sets beyond the list) take that race split over workgroups, where
    the workgroup that ends a race runs the race over p by itself; with the
    bounded-list hint one workgroup runs both.  Both match the oracle."""
    from rejection_sampling_amd import binding as B
    g = np.random.default_rng(3)
    R = 16
    T = g.uniform(0.6, 1.2, size=R).astype(np.float32)
    P = np.where(np.arange(R) % 2 == 0, 1.0, 0.999).astype(np.float32)
    w = W.small_prob_workload(57, R, g.integers(1, 6, size=R), 30011, sigma=1.0, T=T, k=0, P=P)
    qo = w.qo_indptr()
    p = svref.parallel_draft_probs(w.logits, qo, w.temperature, w.top_k, w.top_p, w.request_id,
                                   w.position0, w.seed, THREADS)
    q = (2.0 * p).astype(np.float32)
    d = svref.sample_probs(q, qo, w.request_id, w.position0, w.seed, tag=2)
    ref = oracle_verify(w, qo, d, q, threads=THREADS)
    emitted = np.array([qo[r] + ref["accept_len"][r] for r in range(R)])
    assert np.sum(ref["row_flags"][emitted] & svref.ROW_RESID_EMPTY) >= 4
    for bounded in (False, True):
        progress(f"zero residual, list_bounded={bounded}")
        gpu = gpu_verify(w, qo, d, q, list_bounded=bounded)
        compare_verify(gpu, ref, qo, label=f"zero residual, list_bounded={bounded}")
        assert np.array_equal(gpu["row_flags"] & B.ROW_RESID_EMPTY,
                              ref["row_flags"] & svref.ROW_RESID_EMPTY)


def test_row_order_hint_changes_nothing():
    """Rows of heavy requests scheduled first give the same outputs, bit for
    bit, as the natural order (every result is keyed by request and position),
    and both match the oracle."""
    from rejection_sampling_amd import binding as B
    w = _small(13, 40000, R=24)
    qo = w.qo_indptr()
    q, d = make_drafts(w, qo, THREADS)
    ref = oracle_verify(w, qo, d, q, threads=THREADS)
    prm = params_for(w)
    order = B.heavy_first_order(qo, prm, w.vocab)
    assert order is not None
    outs = []
    for reorder in (False, True):
        progress(f"row order hint, reorder={reorder}")
        call = B.PreparedRejectionSample(dev_logits(w.logits), dev_i32(qo), dev_i32(d), dev_f32(q),
                                         prm, row_order=order if reorder else None)
        o = call()
        torch.cuda.synchronize()
        outs.append({k: v.cpu().numpy() for k, v in o.items()})
    for key in outs[0]:
        assert np.array_equal(outs[0][key], outs[1][key]), key
    compare_verify(outs[1], ref, qo, label="row order")


def _bounded(seed, V, R=32, dtype=W.BF16):
    """Requests whose kept sets are all bounded lists (0 < top-k <= 4096) or
    greedy, with ragged windows."""
    g = np.random.default_rng(seed)
    gam = g.integers(0, 9, size=R)
    T = np.where(g.random(R) < 0.25, 0.0, g.uniform(0.4, 1.3, size=R)).astype(np.float32)
    k = g.choice(np.array([1, 5, 20, 50, 64, 65, 300, 2000], np.int32), size=R)
    P = g.choice(np.array([1.0, 0.95, 0.9, 0.5], np.float32), size=R)
    return W.small_prob_workload(seed, R, gam, V, T=T, k=k, P=P, dtype=dtype)


@pytest.mark.parametrize("V,dtype", [(20007, W.BF16), (9001, W.F32)])
def test_list_bounded_hint_changes_nothing(V, dtype):
    """A batch whose kept sets are all bounded lists (or greedy) gives the same
    outputs, bit for bit, with the list-bounded hint (no split-race launches)
    as without it, with and without a verify cap, and matches the oracle."""
    w = _bounded(31 + V, V, dtype=dtype)
    qo = w.qo_indptr()
    q, d = make_drafts(w, qo, THREADS)
    g = np.random.default_rng(5)
    for cap in (None, np.array([g.integers(-1, x + 2) for x in w.rows_per_request], np.int32)):
        progress(f"list-bounded hint V={V} dtype={dtype} cap={'yes' if cap is not None else 'no'}")
        hinted = gpu_verify(w, qo, d, q, cap, list_bounded=True)
        plain = gpu_verify(w, qo, d, q, cap, list_bounded=False)
        for key in hinted:
            assert np.array_equal(hinted[key], plain[key]), key
        ref = oracle_verify(w, qo, d, q, cap, threads=THREADS)
        compare_verify(hinted, ref, qo, cap=cap, label="list-bounded hint")


def test_wrong_list_bounded_hint():
    """The list-bounded hint claimed for requests with top-k off: their
    correction or bonus token is raced over the whole kept set by one
    workgroup, and matches the oracle and the call without the hint (which
    splits that race over workgroups)."""
    g = np.random.default_rng(77)
    R = 16
    T = g.uniform(0.5, 1.2, size=R).astype(np.float32)
    k = np.where(np.arange(R) % 2 == 0, 0, 20).astype(np.int32)
    P = np.where(np.arange(R) % 4 < 2, 1.0, 0.9).astype(np.float32)
    w = W.small_prob_workload(91, R, g.integers(0, 6, size=R), 12007, T=T, k=k, P=P)
    qo = w.qo_indptr()
    q, d = make_drafts(w, qo, THREADS)
    progress("wrong list-bounded hint")
    hinted = gpu_verify(w, qo, d, q, list_bounded=True)
    plain = gpu_verify(w, qo, d, q, list_bounded=False)
    for key in hinted:
        assert np.array_equal(hinted[key], plain[key]), key
    ref = oracle_verify(w, qo, d, q, threads=THREADS)
    compare_verify(hinted, ref, qo, label="wrong hint")


def test_empty_requests():
    """Requests without rows (leading, between others and trailing) get
    accept_len 0 and next_token -1, with and without the list-bounded hint;
    the other requests match the oracle."""
    import dataclasses
    base = _bounded(55, 9001, R=6)
    layout = [None, 0, None, None, 1, 2, None, 3, 4, 5, None, None]  # None: no rows
    pick = lambda a, fill: np.array([a[x] if x is not None else fill for x in layout], a.dtype)
    w = dataclasses.replace(
        base, num_requests=len(layout),
        temperature=pick(base.temperature, np.float32(0.8)), top_k=pick(base.top_k, np.int32(20)),
        top_p=pick(base.top_p, np.float32(1.0)),
        request_id=np.arange(len(layout), dtype=np.uint32),
        position0=pick(base.position0, np.uint32(0)),
        rows_per_request=pick(base.rows_per_request, np.int32(0)))
    qo = w.qo_indptr()
    q, d = make_drafts(w, qo, THREADS)
    progress("empty requests")
    hinted = gpu_verify(w, qo, d, q, list_bounded=True)
    plain = gpu_verify(w, qo, d, q, list_bounded=False)
    for key in hinted:
        assert np.array_equal(hinted[key], plain[key]), key
    empty = [i for i, x in enumerate(layout) if x is None]
    assert np.all(hinted["accept_len"][empty] == 0) and np.all(hinted["next_token"][empty] == -1)
    ref = oracle_verify(w, qo, d, q, threads=THREADS)
    compare_verify(hinted, ref, qo, label="empty requests")


def test_verify_cap():
    w = _small(7, 12003)
    g = np.random.default_rng(1)
    cap = np.array([g.integers(-1, x + 2) for x in w.rows_per_request], np.int32)
    _run_small(w, verify_cap=cap, label="verify_cap")


def test_tiny_vocabularies():
    for V in (1, 2, 3, 64, 255):
        _run_small(_small(100 + V, V, R=16), label=f"tiny V={V}")


def test_ties_and_quantized_logits():
    """Integer-valued logits: massive ties at the top-k / top-p boundaries and
    top-p rows whose mass lies beyond the candidate buffer (exact path)."""
    w = _small(8, 20000, R=20)
    g = np.random.default_rng(8)
    x = g.integers(0, 8, size=w.logits.shape).astype(np.float32)
    w.logits = W.bf16_bits(x)
    w.draft_logits = W.bf16_bits(x + g.integers(0, 2, size=x.shape).astype(np.float32))
    _run_small(w, label="quantized ties")


def test_minus_inf_and_bad_drafts():
    w = _small(9, 3000, dtype=W.F32, R=16)
    x = W.bf16_to_f32(w.logits) if w.dtype == W.BF16 else w.logits
    x = x.copy()
    x[:, ::7] = -np.inf
    w.logits = x
    qo = w.qo_indptr()
    q, d = make_drafts(w, qo, THREADS)
    d = d.copy()
    d[1::5] = -1
    d[2::9] = w.vocab + 3
    gpu = gpu_verify(w, qo, d, q)
    ref = oracle_verify(w, qo, d, q, threads=THREADS)
    compare_verify(gpu, ref, qo, label="-inf / bad drafts")


def test_all_greedy_without_draft_probs():
    w = W.workload1()
    qo = w.qo_indptr()
    am = svref.parallel_argmax(w.logits, qo)
    d = np.where(w.replace_mask, w.replace_ids, am).astype(np.int32)
    gpu = gpu_verify(w, qo, d, None, all_greedy=True)
    ref = oracle_verify(w, qo, d, None)
    for key in ("accept_len", "next_token", "out_tokens"):
        assert np.array_equal(gpu[key], ref[key]), key


# ------------------------------------------------------- build outputs
def _gpu_build(w, qo, want_probs, kmax):
    from rejection_sampling_amd import binding as B
    out = B.build_target_probs(dev_logits(w.logits), dev_i32(qo), params_for(w),
                               want_probs=want_probs, kmax=kmax)
    diag = B.row_diagnostics(w.num_rows)
    torch.cuda.synchronize()
    gpu = {k: (v.cpu().numpy() if v is not None else None) for k, v in out.items()}
    gpu.update({"diag_" + k: v.cpu().numpy() for k, v in diag.items()})
    return gpu


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_build_target_probs(dtype):
    w = _small(12, 10007, dtype=dtype, R=20)
    qo = w.qo_indptr()
    kmax = 64
    progress(f"build_target_probs dtype={dtype}")
    gpu = _gpu_build(w, qo, True, kmax)
    ref = svref.parallel_build(w.logits, qo, w.temperature, w.top_k, w.top_p, w.request_id,
                               w.position0, w.seed, kmax=kmax, prob_rows=range(w.num_rows),
                               threads=THREADS)
    compare_build(gpu, ref, label="build")


@pytest.mark.parametrize("V", [20000, 32768, 20003])
def test_build_quantized_ties_top_p(V):
    """Integer-valued logits with top-k off and kept sets beyond the list:
    thousands of elements tie at the top-p boundary value, and the kept ones
    are the lowest ids (more ties than the exact path's tie buffer send a row
    to the generic multi-pass kept set).  The dense probabilities of every row
    (zero for a dropped tie) and the kept counts match the oracle, with
    vocabularies of whole 16-byte vectors and one with a scalar tail."""
    g = np.random.default_rng(V)
    R = 12
    T = g.uniform(0.5, 1.5, size=R).astype(np.float32)
    P = np.array([0.3, 0.6, 0.9, 0.999] * 3, np.float32)
    w = W.small_prob_workload(V, R, g.integers(0, 3, size=R), V, T=T, k=0, P=P)
    x = g.integers(0, 8, size=w.logits.shape).astype(np.float32)
    w.logits = W.bf16_bits(x)
    qo = w.qo_indptr()
    kmax = 64
    progress(f"quantized build V={V} rows={w.num_rows}")
    gpu = _gpu_build(w, qo, True, kmax)
    ref = svref.parallel_build(w.logits, qo, w.temperature, w.top_k, w.top_p, w.request_id,
                               w.position0, w.seed, kmax=kmax, prob_rows=range(w.num_rows),
                               threads=THREADS)
    assert int((ref["kept_count"] > 4096).sum()) >= R // 2
    compare_build(gpu, ref, label=f"quantized build V={V}")


def _build_full(w, qo, label, prob_rows):
    """Build parity at a workload's full shape: every row's max, argmax, lse,
    kept count and first 1024 kept ids, dense probabilities on prob_rows, and
    the GPU's Z_K against the oracle's on every sampled row."""
    kmax = 1024
    progress(f"{label}: GPU build ({w.num_rows} rows x {w.vocab})")
    gpu = _gpu_build(w, qo, True, kmax)
    progress(f"{label}: oracle build")
    ref = svref.parallel_build(w.logits, qo, w.temperature, w.top_k, w.top_p, w.request_id,
                               w.position0, w.seed, kmax=kmax, prob_rows=prob_rows,
                               threads=THREADS)
    near, differ = compare_build(gpu, ref, label=label)
    sampled = np.repeat(w.temperature > 0, np.diff(qo))
    zk_err = np.abs(gpu["diag_zk"][sampled] / ref["row_zk"][sampled] - 1.0)
    progress(f"{label}: build ok, near-tie rows {near} (count differs on {differ}), "
             f"max kept {int(gpu['kept_count'].max())}, max |Z_K rel err| {zk_err.max():.3g}")
    assert zk_err.max() < 5e-7


def test_build_full_shape_workload3():
    w = W.workload3()
    qo = w.qo_indptr()
    _build_full(w, qo, "workload 3 build", prob_rows=range(0, w.num_rows, 97))


def test_build_full_shape_workload5():
    w = W.workload5()
    vl, qo, _ = svref.plan_windows(w.confidence, w.budget)
    _build_full(w, qo, "workload 5 build", prob_rows=range(0, w.num_rows, 131))


# ------------------------------------------------------------ workloads
def test_workload1_greedy():
    w = W.workload1()
    qo = w.qo_indptr()
    am = svref.parallel_argmax(w.logits, qo)
    d = np.where(w.replace_mask, w.replace_ids, am).astype(np.int32)
    q = np.zeros((w.num_rows, w.vocab), np.float32)
    q[np.arange(w.num_rows), np.clip(d, 0, w.vocab - 1)] = 1.0
    progress("workload 1 greedy 4x5 V=1024 fp32")
    gpu = gpu_verify(w, qo, d, q)
    ref = oracle_verify(w, qo, d, q)
    for key in ("accept_len", "next_token", "out_tokens"):
        assert np.array_equal(gpu[key], ref[key]), key
    assert np.array_equal(gpu["row_flags"] & 3, ref["row_flags"] & 3)


def test_workload2_full():
    w = W.workload2()
    qo = w.qo_indptr()
    q, d = make_drafts(w, qo, THREADS)
    progress("workload 2 16x6 V=32000")
    gpu = gpu_verify(w, qo, d, q)
    ref = oracle_verify(w, qo, d, q, threads=THREADS)
    compare_verify(gpu, ref, qo, label="workload 2")


def _big(w, qo, label, cap=None):
    progress(f"{label}: drafts by the oracle ({w.num_rows} rows)")
    q, d = make_drafts(w, qo, THREADS)
    progress(f"{label}: GPU verify")
    gpu = gpu_verify(w, qo, d, q, cap, diagnostics=True)
    progress(f"{label}: oracle on every request")
    ref = oracle_verify(w, qo, d, q, cap, threads=THREADS)
    mism, flags = compare_verify(gpu, ref, qo, cap=cap, label=label)
    zk_err, ratio_err, nz, nr = compare_margins(gpu, ref, qo, d, q, label=label)
    progress(f"{label}: margins on {nz} built rows / {nr} tested drafts: max |Z_K rel err| "
             f"{zk_err:.3g}, max |ratio err| {ratio_err:.3g}")
    # properties of every request
    R = w.num_requests
    for r in range(R):
        s, e = qo[r], qo[r + 1]
        L = gpu["accept_len"][r]
        assert 0 <= L <= e - s - 1
        assert gpu["out_tokens"][s + L] == gpu["next_token"][r]
        assert np.array_equal(gpu["out_tokens"][s:s + L], d[s:s + L])
        assert np.all(gpu["out_tokens"][s + L + 1:e] == -1)
        assert 0 <= gpu["next_token"][r] < w.vocab
    progress(f"{label}: ok, mismatches={mism}, flags={flags}, "
             f"mean accepted={gpu['accept_len'].mean():.3f}")
    return gpu, q, d


def test_workload3_full():
    w = W.workload3()
    qo = w.qo_indptr()
    _big(w, qo, "workload 3 128x8 V=248320")


def test_workload4_full():
    w = W.workload4()
    qo = w.qo_indptr()
    greedy = np.nonzero(w.temperature == 0)[0]
    gpu, q, d = _big(w, qo, "workload 4 512x8 V=129280")
    # greedy requests of the whole batch: emitted token is the row argmax
    x = W.bf16_to_f32(w.logits)
    for r in greedy:
        s = qo[r]
        L = gpu["accept_len"][r]
        assert gpu["next_token"][r] == int(np.argmax(x[s + L]))


def test_workload5_planner_and_verify():
    w = W.workload5()
    from rejection_sampling_amd import binding as B
    progress("workload 5 planner")
    vl_g, qo_g, surv_g = B.plan_windows(dev_f32(w.confidence), w.budget)
    torch.cuda.synchronize()
    vl, qo, surv = svref.plan_windows(w.confidence, w.budget)
    assert np.array_equal(vl_g.cpu().numpy(), vl)
    assert np.array_equal(qo_g.cpu().numpy(), qo)
    assert np.array_equal(surv_g.cpu().numpy().view(np.uint32), surv.view(np.uint32))
    assert qo[-1] == w.num_rows
    gpu, _, _ = _big(w, qo, "workload 5 ragged 1792 rows V=248320")
    # the step's acceptance and trim statistics over the planner's windows
    Bk = w.confidence.shape[1]
    st_g = B.acceptance_stats(dev_i32(gpu["accept_len"]), vl_g, Bk).cpu().numpy()
    st = svref.acceptance_stats(gpu["accept_len"], vl, Bk)
    assert np.array_equal(st_g, st)
    progress(f"workload 5 statistics: trimmed {st[1]}/{st[0]}, regret {st[2]}, "
             f"acceptance per verified token {st[3] / max(st[4], 1):.3f}")


# -------------------------------------------------------------- planner
@pytest.mark.parametrize("R,Bk", [(1, 1), (7, 3), (256, 16), (1024, 8), (1000, 9), (3000, 2), (100, 20)])
def test_planner_matches_oracle(R, Bk):
    from rejection_sampling_amd import binding as B
    g = np.random.default_rng(R)
    conf = g.random((R, Bk)).astype(np.float32)
    conf[g.random((R, Bk)) < 0.02] = np.nan
    conf[g.random((R, Bk)) < 0.02] = 1.5
    for budget in (-3, 0, 1, R * Bk // 3, R * Bk - 1, R * Bk, R * Bk + 5):
        vl_g, qo_g, surv_g = B.plan_windows(dev_f32(conf), budget)
        vl, qo, surv = svref.plan_windows(conf, budget)
        assert np.array_equal(vl_g.cpu().numpy(), vl), budget
        assert np.array_equal(qo_g.cpu().numpy(), qo), budget
        assert np.array_equal(surv_g.cpu().numpy().view(np.uint32), surv.view(np.uint32))
    # all-equal confidences: pure index tie-break
    conf = np.full((R, Bk), 0.5, np.float32)
    vl_g, qo_g, _ = B.plan_windows(dev_f32(conf), (R * Bk) // 2 + 1)
    vl, qo, _ = svref.plan_windows(conf, (R * Bk) // 2 + 1)
    assert np.array_equal(vl_g.cpu().numpy(), vl)
    # confidences a few ulps below 1: survivals share their leading key bytes
    conf = (1.0 - g.integers(1, 6, (R, Bk)) * 2.0 ** -24).astype(np.float32)
    for budget in (1, R * Bk // 2, R * Bk - 1):
        vl_g, _, _ = B.plan_windows(dev_f32(conf), budget)
        vl, _, _ = svref.plan_windows(conf, budget)
        assert np.array_equal(vl_g.cpu().numpy(), vl), budget


@pytest.mark.parametrize("R,Bk", [(0, 5), (1, 0), (3, 1), (256, 16), (5000, 7), (300, 1024)])
def test_acceptance_stats_match_oracle(R, Bk):
    """Acceptance and trim statistics bit-exact against the oracle, with
    out-of-range device values (clamped alike on both sides)."""
    from rejection_sampling_amd import binding as B
    g = np.random.default_rng(R + 7 * Bk)
    w = g.integers(-2, Bk + 3, R).astype(np.int32)
    L = g.integers(-2, Bk + 3, R).astype(np.int32)
    full = g.random(R) < 0.3                      # some requests accept their whole window
    L[full] = w[full]
    progress(f"acceptance statistics R={R} B={Bk}")
    st_g = B.acceptance_stats(dev_i32(L) if R else torch.empty(0, dtype=torch.int32, device="cuda"),
                              dev_i32(w) if R else torch.empty(0, dtype=torch.int32, device="cuda"),
                              Bk).cpu().numpy()
    assert np.array_equal(st_g, svref.acceptance_stats(L, w, Bk))


def test_estimator_predict_matches_oracle():
    """Features and confidences of the online acceptance estimator from the
    library's own draft build (row max, lse), against the oracle's feature and
    prediction on the same arrays."""
    from rejection_sampling_amd import binding as B
    R, Bk, V = 40, 6, 3001
    g = np.random.default_rng(21)
    x = (g.normal(0, 3, (R * Bk, V))).astype(np.float32)
    x[3, 17] = 60.0                                   # a row with q_max = 1 in fp32 terms
    T = g.uniform(0.4, 1.3, R).astype(np.float32)
    T[::4] = 0.0                                      # greedy requests
    qo = (np.arange(R + 1) * Bk).astype(np.int32)
    prm = B.Params(dev_f32(T), None, None)
    built = B.build_target_probs(dev_f32(x), dev_i32(qo), prm)
    m, lse = built["row_max"], built["row_lse"]
    est = B.AcceptanceEstimator(Bk)
    progress(f"estimator predict R={R} B={Bk}")
    feat_g, conf_g = est.predict(m, lse, dev_f32(T))
    t_eff = np.repeat(T, Bk)
    feat = svref.est_feature(m.cpu().numpy(), lse.cpu().numpy(), t_eff)
    fg = feat_g.cpu().numpy().reshape(-1)
    # compared as probabilities: logit is ill-conditioned as q_max nears 1, where
    # one ulp of exp on either side moves x by ~1e-16 / (1 - q_max)
    expit = lambda v: 1.0 / (1.0 + np.exp(-v))
    assert np.allclose(expit(fg), expit(feat), rtol=0, atol=1e-13)
    mid = np.abs(feat) < 20
    assert np.allclose(fg[mid], feat[mid], rtol=1e-11, atol=1e-11)
    ref = svref.Estimator(Bk)
    p = ref.predict(feat, np.tile(np.arange(Bk, dtype=np.int32), R))
    assert np.allclose(conf_g.cpu().numpy().reshape(-1), p.astype(np.float32), rtol=2e-7, atol=0)


def test_estimator_observe_and_refit_match_oracle():
    """250 observed steps (two refits) on simulated drafts: the device state's
    coefficients follow the oracle's within rounding (its sums run in another
    order), and the same inputs give the same device state twice."""
    from rejection_sampling_amd import binding as B
    R, Bk = 96, 8
    g = np.random.default_rng(22)
    true_b = np.linspace(1.0, -1.5, Bk)
    steps = []
    for _ in range(250):
        xs = g.normal(0, 2, (R, Bk))
        p = 1 / (1 + np.exp(-(1.0 * xs + true_b)))
        surv = g.random((R, Bk)) < p
        L = np.where(surv.all(axis=1), Bk, np.argmin(surv, axis=1)).astype(np.int32)
        w = g.integers(0, Bk + 1, R).astype(np.int32)
        steps.append((xs, np.minimum(L, w), w))
    states = []
    for rep in range(2):
        est = B.AcceptanceEstimator(Bk)
        ref = svref.Estimator(Bk)
        progress(f"estimator observe, pass {rep}")
        for c, (xs, L, w) in enumerate(steps):
            est.observe(torch.from_numpy(xs).cuda(), dev_i32(L), dev_i32(w))
            ref.observe(xs, L, w)
            if (c + 1) % 50 == 0:
                s, b, n = est.coefficients()
                assert n == ref.st.refits
                assert s == pytest.approx(ref.slope, rel=1e-9, abs=1e-12)
                assert np.allclose(b, ref.bias, rtol=1e-9, atol=1e-12)
        states.append(est.state.cpu().numpy())
    assert ref.st.refits == 2
    assert np.array_equal(states[0].view(np.uint64), states[1].view(np.uint64))


def test_estimator_observe_wide_block_matches_oracle():
    """Blocks wider than the workgroup's 16 waves (several positions per wave)
    and more requests than one load round: one refit after 100 steps."""
    from rejection_sampling_amd import binding as B
    R, Bk = 700, 40
    g = np.random.default_rng(23)
    true_b = np.linspace(2.0, -2.0, Bk)
    est = B.AcceptanceEstimator(Bk)
    ref = svref.Estimator(Bk)
    progress(f"estimator observe R={R} B={Bk}")
    for c in range(110):
        xs = g.normal(0, 2, (R, Bk))
        surv = g.random((R, Bk)) < 1 / (1 + np.exp(-(0.8 * xs + true_b)))
        L = np.where(surv.all(axis=1), Bk, np.argmin(surv, axis=1)).astype(np.int32)
        w = g.integers(-1, Bk + 2, R).astype(np.int32)
        L = np.minimum(L, np.maximum(w, 0)).astype(np.int32)
        est.observe(torch.from_numpy(xs).cuda(), dev_i32(L), dev_i32(w))
        ref.observe(xs, L, w)
    s_, b, n = est.coefficients()
    assert n == ref.st.refits == 1
    assert s_ == pytest.approx(ref.slope, rel=1e-9, abs=1e-12)
    assert np.allclose(b, ref.bias, rtol=1e-9, atol=1e-12)


def test_accept_prefix_matches_oracle():
    from rejection_sampling_amd import binding as B
    g = np.random.default_rng(3)
    R = 300
    lens = g.integers(1, 80, size=R)
    qo = np.zeros(R + 1, np.int32)
    np.cumsum(lens, out=qo[1:])
    acc = (g.random(qo[-1]) < 0.9).astype(np.uint8)
    cap = g.integers(-2, 90, size=R).astype(np.int32)
    for c in (None, cap):
        got = B.accept_prefix(torch.from_numpy(acc).cuda(), dev_i32(qo),
                              dev_i32(c) if c is not None else None).cpu().numpy()
        assert np.array_equal(got, svref.accept_prefix(acc, qo, c))


# -------------------------------------------------- distribution on GPU
def test_gpu_first_token_chi_square():
    """The GPU's first emitted token follows the target (chi-square, 10^6
    trials of one request each, V = 64)."""
    from scipy import stats
    from rejection_sampling_amd import binding as B
    g = np.random.default_rng(101)
    V, n = 64, 1_000_000
    x = g.normal(0, 1.5, size=(2, V)).astype(np.float32)
    xd = (x + g.normal(0, 1.0, size=x.shape)).astype(np.float32)
    q1 = svref.build_target_probs(xd, np.array([0, 2], np.int32), np.ones(1, np.float32),
                                  want_probs=True)["probs"].astype(np.float32)
    p0 = svref.build_target_probs(x[:1], np.array([0, 1], np.int32), np.ones(1, np.float32),
                                  want_probs=True)["probs"][0]
    qo = np.arange(n + 1, dtype=np.int32) * 2
    rid = np.arange(n, dtype=np.uint32)
    pos0 = np.zeros(n, np.uint32)
    q = np.ascontiguousarray(np.broadcast_to(q1, (n, 2, V))).reshape(2 * n, V)
    d = svref.sample_probs(q, qo, rid, pos0, 77, tag=2)
    logits = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(x, (n, 2, V))).reshape(2 * n, V)).cuda()
    prm = B.Params(dev_f32(np.ones(n)), None, None, dev_i32(rid), dev_i32(pos0), 77)
    progress("GPU chi-square 10^6 trials")
    out = B.rejection_sample(logits, dev_i32(qo), dev_i32(d), dev_f32(q), prm)
    first = out["out_tokens"].view(n, 2)[:, 0].cpu().numpy()
    counts = np.bincount(first, minlength=V)
    exp = n * p0
    chi2 = ((counts - exp) ** 2 / exp).sum()
    assert stats.chi2.sf(chi2, V - 1) > 0.01
