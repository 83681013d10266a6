"""Pins of the oracle's target-distribution build.

What the pages fix ("Adaptive verification for DFLASH", commit note on
build_speculative_verify_target_probs): top-k is taken on the raw logits and
only the selected values are divided by the temperature, because a positive
temperature keeps the order; the kept count and probability values do not
depend on how ties at the top-k boundary are broken.  The consolidation study
(section 2) fixes greedy as the argmax.  Pins here are library routines (numpy
argmax / lexsort, scipy softmax / logsumexp) and brute force over subsets for
the nucleus, none of which share the oracle's code path.
"""
import itertools

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

from rejection_sampling_amd.workloads import bf16_bits, bf16_to_f32


def one_request(rows):
    return np.array([0, rows], np.int32)


def quantized_rows(g, rows, V, levels=8):
    return g.integers(0, levels, size=(rows, V)).astype(np.float32)


def test_greedy_argmax_is_numpy_first_occurrence(oracle):
    g = np.random.default_rng(1)
    x = quantized_rows(g, 64, 257)          # heavy ties
    y = g.normal(0, 3, size=(64, 1000)).astype(np.float32)
    for logits in (x, y):
        out = oracle.build_target_probs(logits, one_request(len(logits)),
                                        np.zeros(1, np.float32), kmax=1)
        assert np.array_equal(out["row_argmax"], np.argmax(logits, axis=1))
        assert np.array_equal(out["row_max"], logits.max(axis=1).astype(np.float64))
        assert np.all(out["kept_count"] == 1)


def test_bf16_rows_read_exactly(oracle):
    g = np.random.default_rng(2)
    bits = bf16_bits(g.normal(0, 4, size=(8, 333)).astype(np.float32))
    vals = bf16_to_f32(bits)
    out = oracle.build_target_probs(bits, one_request(8), np.zeros(1, np.float32))
    assert np.array_equal(out["row_max"], vals.max(axis=1).astype(np.float64))
    assert np.array_equal(out["row_argmax"], np.argmax(vals, axis=1))


@pytest.mark.parametrize("T", [0.3, 0.7, 1.0, 1.9])
def test_topk_V_topp_1_is_plain_softmax(oracle, T):
    g = np.random.default_rng(3)
    logits = g.normal(0, 3, size=(6, 500)).astype(np.float32)
    for k in (0, 500, 10**6):
        out = oracle.build_target_probs(logits, one_request(6), np.array([T], np.float32),
                                        np.array([k], np.int32), np.array([1.0], np.float32),
                                        want_probs=True)
        T64 = float(np.float32(T))      # temperatures are fp32 inputs
        ref = softmax(logits.astype(np.float64) / T64, axis=1)
        np.testing.assert_allclose(out["probs"], ref, rtol=1e-12, atol=1e-300)
        assert np.all(out["kept_count"] == 500)


@pytest.mark.parametrize("T", [0.5, 1.0])
def test_lse_matches_scipy(oracle, T):
    g = np.random.default_rng(4)
    logits = g.normal(0, 4, size=(5, 2000)).astype(np.float32)
    out = oracle.build_target_probs(logits, one_request(5), np.array([T], np.float32))
    ref = logsumexp(logits.astype(np.float64) / float(np.float32(T)), axis=1)
    np.testing.assert_allclose(out["row_lse"], ref, rtol=0, atol=1e-10)
    # greedy rows report lse at T = 1
    out0 = oracle.build_target_probs(logits, one_request(5), np.zeros(1, np.float32))
    np.testing.assert_allclose(out0["row_lse"], logsumexp(logits.astype(np.float64), axis=1),
                               rtol=0, atol=1e-10)


@pytest.mark.parametrize("k", [1, 2, 7, 20, 50, 255])
def test_topk_sets_match_lexsort(oracle, k):
    g = np.random.default_rng(5 + k)
    for logits in (quantized_rows(g, 16, 256), g.normal(0, 3, size=(16, 256)).astype(np.float32)):
        out = oracle.build_target_probs(logits, one_request(16), np.array([0.9], np.float32),
                                        np.array([k], np.int32), np.array([1.0], np.float32),
                                        kmax=k, want_probs=True)
        assert np.all(out["kept_count"] == k)
        for i, row in enumerate(logits):
            order = np.lexsort((np.arange(len(row)), -row.astype(np.float64)))
            assert np.array_equal(out["kept_idx"][i], order[:k])
            # probabilities: softmax over the kept values only (any tie choice
            # gives the same values -- the page's claim)
            ref = softmax(row[order[:k]].astype(np.float64) / float(np.float32(0.9)))
            np.testing.assert_allclose(out["probs"][i][order[:k]], ref, rtol=1e-12)
            assert np.all(out["probs"][i][order[k:]] == 0.0)


def test_topk_values_independent_of_tie_choice(oracle):
    """Permuting the vocabulary changes which tied ids are kept, never the kept
    count or the multiset of kept probabilities."""
    g = np.random.default_rng(6)
    x = quantized_rows(g, 4, 64, levels=5)
    perm = g.permutation(64)
    a = oracle.build_target_probs(x, one_request(4), np.array([1.3], np.float32),
                                  np.array([10], np.int32), want_probs=True)
    b = oracle.build_target_probs(x[:, perm], one_request(4), np.array([1.3], np.float32),
                                  np.array([10], np.int32), want_probs=True)
    assert np.array_equal(a["kept_count"], b["kept_count"])
    for i in range(4):
        np.testing.assert_allclose(np.sort(a["probs"][i]), np.sort(b["probs"][i]), rtol=1e-14)


def _nucleus_bruteforce(p, P):
    """Smallest set of tokens whose mass reaches P (Holtzman et al.): search
    over all subsets by size; the minimum size n is reached by the n most
    probable tokens.  Returns n."""
    V = len(p)
    for n in range(1, V + 1):
        best = max(sum(p[list(c)]) for c in itertools.combinations(range(V), n))
        if best >= float(np.float32(P)) * (1 - 1e-15) * p.sum():
            return n
    return V


@pytest.mark.parametrize("P", [0.05, 0.3, 0.5, 0.8, 0.9, 0.97])
def test_topp_is_smallest_set_reaching_p(oracle, P):
    g = np.random.default_rng(int(P * 1000))
    V = 11
    for trial in range(6):
        x = g.normal(0, 2, size=V).astype(np.float32)
        out = oracle.build_target_probs(x[None, :], one_request(1), np.array([1.0], np.float32),
                                        None, np.array([P], np.float32), kmax=V,
                                        want_probs=True)
        p = softmax(x.astype(np.float64))
        n = _nucleus_bruteforce(p, P)
        assert out["kept_count"][0] == n
        kept = out["kept_idx"][0][:n]
        order = np.lexsort((np.arange(V), -x.astype(np.float64)))
        assert np.array_equal(kept, order[:n])
        np.testing.assert_allclose(out["probs"][0][kept], p[kept] / p[kept].sum(), rtol=1e-12)


def test_topk_then_topp_mass_invariants(oracle):
    g = np.random.default_rng(8)
    logits = g.normal(0, 3, size=(40, 3000)).astype(np.float32)
    T, k, P = 0.7, 50, 0.9
    out = oracle.build_target_probs(logits, one_request(40), np.array([T], np.float32),
                                    np.array([k], np.int32), np.array([P], np.float32),
                                    kmax=k, want_probs=True)
    for i, row in enumerate(logits):
        order = np.lexsort((np.arange(len(row)), -row.astype(np.float64)))
        pk = softmax(row[order[:k]].astype(np.float64) / float(np.float32(T)))  # top-k renorm.
        n = out["kept_count"][i]
        assert 1 <= n <= k
        P32 = float(np.float32(P))
        assert pk[: n - 1].sum() < P32 <= pk[:n].sum() + 1e-12
        assert np.array_equal(out["kept_idx"][i][:n], order[:n])
        np.testing.assert_allclose(out["probs"][i].sum(), 1.0, rtol=1e-12)


def test_topp_edge_values(oracle):
    g = np.random.default_rng(9)
    x = g.normal(0, 2, size=(3, 100)).astype(np.float32)
    for P, want in ((0.0, 1), (-1.0, 1), (1.0, 100), (1.5, 100), (float("nan"), 100)):
        out = oracle.build_target_probs(x, one_request(3), np.array([1.0], np.float32), None,
                                        np.array([P], np.float32))
        assert np.all(out["kept_count"] == want), P


def test_minus_inf_logits_get_zero_mass(oracle):
    x = np.array([[0.0, -np.inf, 1.0, -np.inf, 2.0]], np.float32)
    out = oracle.build_target_probs(x, one_request(1), np.array([1.0], np.float32),
                                    want_probs=True)
    p = out["probs"][0]
    assert p[1] == 0 and p[3] == 0
    np.testing.assert_allclose(p[[0, 2, 4]], softmax([0.0, 1.0, 2.0]), rtol=1e-14)
