"""Pins of the oracle's confidence planner.

TensorRT-LLM PR #17056 (first commit note and description): a position's
survival is the running product of its request's confidences; one batch-wide
ranking by survival, ties ordered by position and request, decides the verified
positions; windows are packed with a qo_indptr, one bonus row per request (review-pass note:
tokens submitted are verify_len + 1 per request).  The consolidation study's
section 1 prints per-position acceptance and accepted tokens per draft, whose
relation (expected accepted length = sum of survivals) is the planner's
objective.

Pins: O(N^2) rank counting without any sort, exhaustive search over every
allocation for small cases (the rank allocation maximises total survival), the
printed acceptance figures, and edge cases.
"""
import itertools
import os

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def _survival_f32(conf):
    c = np.where(conf > 0, np.minimum(conf, 1), 0).astype(np.float32)
    c[np.isnan(conf)] = 0
    S = np.empty_like(c)
    for r in range(c.shape[0]):
        acc = np.float32(1)
        for j in range(c.shape[1]):
            acc = c[r, j] if j == 0 else np.float32(acc * c[r, j])
            S[r, j] = acc
    return S


def _rank_count_lengths(S, budget):
    """verify_len by counting, for every (r, j), how many items beat it under
    (S desc, j asc, r asc); selected iff that count < budget."""
    R, B = S.shape
    s = S.reshape(-1).astype(np.float64)
    j = np.tile(np.arange(B), R)
    r = np.repeat(np.arange(R), B)
    beats = (s[None, :] > s[:, None]) | ((s[None, :] == s[:, None]) & (
        (j[None, :] < j[:, None]) | ((j[None, :] == j[:, None]) & (r[None, :] < r[:, None]))))
    rank = beats.sum(axis=1)
    sel = rank < budget
    return np.bincount(r[sel], minlength=R).astype(np.int32)


def test_survival_is_fp32_left_to_right_cumprod(oracle):
    g = np.random.default_rng(1)
    conf = g.random((20, 16)).astype(np.float32)
    conf[3, 5] = np.nan
    conf[4, 2] = -0.5
    conf[5, 7] = 1.7
    _, _, surv = oracle.plan_windows(conf, 40)
    assert np.array_equal(surv, _survival_f32(conf))


@pytest.mark.parametrize("R,B", [(1, 4), (3, 5), (8, 4), (37, 16), (256, 16)])
def test_rank_allocation_matches_counting(oracle, R, B):
    g = np.random.default_rng(R * 100 + B)
    z = g.normal(1.0, 1.5, size=(R, B))
    conf = (1 / (1 + np.exp(-z)) * 0.95 ** np.arange(B)).astype(np.float32)
    for budget in (0, 1, R, R * B // 3, R * B - 1, R * B, R * B + 7):
        vl, qo, surv = oracle.plan_windows(conf, budget)
        want = _rank_count_lengths(_survival_f32(conf), budget)
        assert np.array_equal(vl, want), budget
        assert vl.sum() == min(budget, R * B)
        assert qo[0] == 0 and np.array_equal(np.diff(qo), vl + 1)
        assert qo[-1] == min(budget, R * B) + R


def test_rank_allocation_is_optimal_exhaustively(oracle):
    """For <= 8 requests x B <= 4, every allocation with sum(len) <= budget is
    enumerated; the rank allocation attains the maximum total survival."""
    g = np.random.default_rng(7)
    for trial in range(6):
        R, B = (8, 4) if trial < 3 else (5, 3)
        conf = g.random((R, B)).astype(np.float32) ** 0.5
        S = _survival_f32(conf).astype(np.float64)
        prefix = np.concatenate([np.zeros((R, 1)), np.cumsum(S, axis=1)], axis=1)
        for budget in (3, 9, 14):
            vl, _, _ = oracle.plan_windows(conf, budget)
            got = prefix[np.arange(R), vl].sum()
            best = -1.0
            for alloc in itertools.product(range(B + 1), repeat=R):
                if sum(alloc) <= budget:
                    best = max(best, prefix[np.arange(R), list(alloc)].sum())
            assert abs(got - best) <= 1e-12 * max(1.0, best)


def test_all_equal_confidence_uses_index_tie_break(oracle):
    R, B = 10, 6
    conf = np.full((R, B), 0.5, np.float32)
    # S depends on j only: ties across requests at each j resolve by r asc
    vl, _, _ = oracle.plan_windows(conf, 23)
    assert list(vl) == [3, 3, 3] + [2] * 7
    conf1 = np.ones((R, B), np.float32)   # every S == 1: pure (j, r) order
    vl1, _, _ = oracle.plan_windows(conf1, 23)
    assert list(vl1) == [3, 3, 3] + [2] * 7


def test_budget_edges_and_underflow(oracle):
    g = np.random.default_rng(9)
    conf = (g.random((12, 16)) * 1e-6).astype(np.float32)   # survivals underflow
    for budget in (-5, 0, 50, 12 * 16, 10**6):
        vl, qo, surv = oracle.plan_windows(conf, budget)
        assert vl.sum() == max(0, min(budget, 12 * 16))
        assert np.array_equal(vl, _rank_count_lengths(_survival_f32(conf), max(0, budget)))
    assert np.any(surv == 0)


def test_windows_are_prefixes(oracle):
    g = np.random.default_rng(10)
    conf = g.random((64, 16)).astype(np.float32)
    vl, _, surv = oracle.plan_windows(conf, 300)
    # the selection is {S > s*} plus part of {S == s*}: each request's selected
    # positions form a prefix because S is non-increasing along j
    assert np.all(np.diff(surv, axis=1) <= 0)
    thr = np.sort(surv.reshape(-1))[::-1][299]
    for r in range(64):
        assert np.all(surv[r, : vl[r]] >= thr)
        assert np.all(surv[r, vl[r]:] <= thr)


def test_printed_acceptance_is_sum_of_survivals(oracle):
    """The study's per-position acceptance figures are prefix survivals; their
    sum is the printed accepted-per-draft figure (the planner's objective)."""
    vals = {}
    with open(os.path.join(HERE, "golden", "per_position_acceptance.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            key, *rest = line.split()
            vals[key] = [float(t) for t in rest]
    S = np.array(vals["survival"])
    conf = np.empty((1, 5), np.float32)
    conf[0, 0] = S[0]
    conf[0, 1:] = S[1:] / S[:-1]          # per-position conditional acceptance
    _, _, surv = oracle.plan_windows(conf, 5)
    np.testing.assert_allclose(surv[0], S, rtol=1e-6)
    accepted_per_draft = vals["accepted_tokens"][0] / vals["drafts"][0]
    assert abs(accepted_per_draft - vals["accepted_per_draft"][0]) < 0.005
    assert abs(surv[0].sum() - accepted_per_draft) < 0.002
    assert abs(surv[0].sum() / 5 - vals["acceptance_per_draft_token"][0]) < 0.001
