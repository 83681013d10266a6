"""GPU parity of block verification (SV_BLOCK_VERIFY) against the CPU oracle.

Block verification (Sun et al., "Block Verification Accelerates Speculative
Decoding"; the consolidation study's rejection_sample_method "block") runs in
the request finalize on the row pass's kept lists.  Every case compares every
request with the oracle's block rule under the near-tie rules; one drafted
position must equal the device's own token rule bit for bit; the first
emitted token must follow the target (chi-square over 10^6 one-request
trials); and the full-size top-k and top-p workloads are compared whole.
"""
import os

import numpy as np
import pytest
import torch

from oracle import svref
from rejection_sampling_amd import workloads as W
from tests.gpu_common import (compare_verify, dev_f32, dev_i32, gpu_verify, make_drafts,
                              oracle_verify, progress)

pytestmark = pytest.mark.gpu

THREADS = min(16, os.cpu_count() or 1)

GRID = [(0.0, 0, 1.0), (0.8, 0, 1.0), (0.8, 0, 0.9), (1.0, 20, 0.95), (0.7, 50, 0.9),
        (1.3, 5, 1.0), (0.5, 1, 0.5), (1.0, 2000, 0.9), (0.9, 0, 0.0), (1.2, 300, 0.97)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from rejection_sampling_amd import binding
    binding.load()
    yield


def _grid(seed, V, R=24, dtype=W.BF16, gmax=8, noise=1.0):
    g = np.random.default_rng(seed)
    c = g.integers(0, len(GRID), size=R)
    T = np.array([GRID[i][0] for i in c], np.float32)
    k = np.array([GRID[i][1] for i in c], np.int32)
    P = np.array([GRID[i][2] for i in c], np.float32)
    return W.small_prob_workload(seed, R, g.integers(0, gmax, size=R), V, T=T, k=k, P=P,
                                 dtype=dtype, noise=noise)


def _check(w, label, cap=None, list_bounded=None):
    qo = w.qo_indptr()
    q, d = make_drafts(w, qo, THREADS)
    progress(f"{label}: rows={w.num_rows} V={w.vocab}")
    gpu = gpu_verify(w, qo, d, q, cap, block=True, list_bounded=list_bounded)
    ref = oracle_verify(w, qo, d, q, cap, threads=THREADS, block=True)
    mism, flags = compare_verify(gpu, ref, qo, cap=cap, label=label, block=True)
    for r in range(w.num_requests):
        s, e = qo[r], qo[r + 1]
        L = gpu["accept_len"][r]
        assert gpu["out_tokens"][s + L] == gpu["next_token"][r]
        assert np.array_equal(gpu["out_tokens"][s:s + L], d[s:s + L])
    return gpu, ref


@pytest.mark.parametrize("V,dtype", [(20007, W.BF16), (32000, W.BF16), (9001, W.F32)])
def test_block_grid(V, dtype):
    _check(_grid(71 + V, V, dtype=dtype), f"block grid V={V}")


def test_block_noisy_drafts_and_cap():
    w = _grid(72, 12003, noise=2.5)
    g = np.random.default_rng(2)
    cap = np.array([g.integers(-1, x + 2) for x in w.rows_per_request], np.int32)
    _check(w, "block with a verify cap", cap=cap)


def test_block_whole_row_kept_sets_split_and_single():
    """Requests with top-k and top-p off (whole-row kept sets: the test bound
    and the residual race over the whole row), with the split race and with
    the one-workgroup race."""
    g = np.random.default_rng(73)
    R = 12
    T = g.uniform(0.5, 1.2, R).astype(np.float32)
    k = np.where(np.arange(R) % 2 == 0, 0, 20).astype(np.int32)
    w = W.small_prob_workload(73, R, g.integers(1, 6, size=R), 40000, T=T, k=k, P=1.0)
    for bounded in (False, True):
        _check(w, f"block whole rows list_bounded={bounded}", list_bounded=bounded)


def test_block_one_position_is_the_token_rule():
    w = _grid(74, 20007, R=40)          # the grid's sampling values
    w2 = W.small_prob_workload(74, 40, 1, 20007, T=w.temperature, k=w.top_k, P=w.top_p)
    qo = w2.qo_indptr()
    q, d = make_drafts(w2, qo, THREADS)
    progress("block, one drafted position, against the token rule")
    a = gpu_verify(w2, qo, d, q, block=False)
    b = gpu_verify(w2, qo, d, q, block=True)
    for key in ("accept_len", "out_tokens", "next_token", "row_flags"):
        assert np.array_equal(a[key], b[key]), key


def test_block_workload3_full():
    w = W.workload3()
    gpu, ref = _check(w, "block workload 3 128x8 V=248320")
    progress(f"block workload 3: mean accepted {gpu['accept_len'].mean():.3f}")


def test_block_workload5_full():
    w = W.workload5()
    vl, qo, _ = svref.plan_windows(w.confidence, w.budget)
    w.rows_per_request = (vl + 1).astype(np.int32)
    gpu, ref = _check(w, "block workload 5 ragged V=248320")
    progress(f"block workload 5: mean accepted {gpu['accept_len'].mean():.3f}")


def test_gpu_block_first_token_chi_square():
    """The GPU's first emitted token under block verification follows the
    target: 10^6 one-request trials, 3 drafted positions, V = 64."""
    from scipy import stats
    from rejection_sampling_amd import binding as B
    g = np.random.default_rng(103)
    V, n, gam = 64, 1_000_000, 3
    x = g.normal(0, 1.5, size=(gam + 1, V)).astype(np.float32)
    xd = (x + g.normal(0, 1.0, size=x.shape)).astype(np.float32)
    q1 = svref.build_target_probs(xd, np.array([0, gam + 1], np.int32), np.ones(1, np.float32),
                                  want_probs=True)["probs"].astype(np.float32)
    p0 = svref.build_target_probs(x[:1], np.array([0, 1], np.int32), np.ones(1, np.float32),
                                  want_probs=True)["probs"][0]
    qo = np.arange(n + 1, dtype=np.int32) * (gam + 1)
    rid = np.arange(n, dtype=np.uint32)
    pos0 = np.zeros(n, np.uint32)
    q = np.ascontiguousarray(np.broadcast_to(q1, (n, gam + 1, V))).reshape(n * (gam + 1), V)
    d = svref.sample_probs(q, qo, rid, pos0, 78, tag=2)
    logits = torch.from_numpy(
        np.ascontiguousarray(np.broadcast_to(x, (n, gam + 1, V))).reshape(n * (gam + 1), V)).cuda()
    prm = B.Params(dev_f32(np.ones(n)), None, None, dev_i32(rid), dev_i32(pos0), 78, block=True)
    progress("GPU block chi-square 10^6 trials")
    out = B.rejection_sample(logits, dev_i32(qo), dev_i32(d), dev_f32(q), prm)
    first = out["out_tokens"].view(n, gam + 1)[:, 0].cpu().numpy()
    L = out["accept_len"].cpu().numpy()
    # the same outputs as the oracle's block rule on the first 20000 trials
    m = 20000
    ref = svref.parallel_rejection_sample(x[np.tile(np.arange(gam + 1), m)], qo[:m + 1], d[:m * (gam + 1)],
                                          q[:m * (gam + 1)], np.ones(m, np.float32), None, None,
                                          rid[:m], pos0[:m], 78, block=True, threads=THREADS)
    assert np.array_equal(L[:m], ref["accept_len"])
    assert np.array_equal(first[:m], ref["out_tokens"].reshape(m, gam + 1)[:, 0])
    counts = np.bincount(first, minlength=V)
    exp = n * p0
    chi2 = ((counts - exp) ** 2 / exp).sum()
    assert stats.chi2.sf(chi2, V - 1) > 0.01
    progress(f"block chi-square ok, mean accepted {L.mean():.4f}")
