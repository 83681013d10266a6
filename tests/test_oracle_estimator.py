"""Pins of the oracle's online acceptance estimator.

SGLang PR "Adaptive verification for DFLASH ... built on upstream DSpark",
commit notes adding OnlineAcceptanceEstimator and fixing its slope refit:
p_k = sigmoid(slope * x_k + bias_k) with x_k = logit(q_max) of the
temperature-scaled draft distribution (greedy rows at T = 1, clamped to
+-40); slope 0.5 and intercepts -0.2 at the start; observe() labels the
accepted drafts and the first rejected one; every 100 calls an arrowhead
Newton (IRLS) solve with ridge 1e-3, updates damped by n / (n + 50),
non-finite steps dropped, a slope step that would turn the slope negative
halved at most 8 times (dropped if it still crosses zero), intercepts stepped
given the slope step taken.  The fix's note reports the slope reaching 0.96
within ten refits from 3.0 on drafts generated with slope 1.0, and 0 to 0.06
from the default start on drafts whose feature carries no signal.

Pins: the feature against scipy's logsumexp and logit; the Newton direction
against numpy's dense solve of the full (B+1)-square system; recovery of the
generating coefficients from simulated drafts; the two behaviours the fix
reports; the slope never negative; the start values.
"""
import numpy as np
import pytest
from scipy.special import logit, logsumexp

from oracle import svref


def test_start_values():
    est = svref.Estimator(5)
    assert est.slope == 0.5 and np.all(est.bias == -0.2)


def test_feature_is_logit_of_the_softmax_max():
    rng = np.random.default_rng(0)
    rows, V = 40, 300
    x = rng.normal(0, 3, (rows, V)).astype(np.float32)
    T = rng.uniform(0.3, 1.5, rows).astype(np.float32)
    T[::5] = 0.0                                         # greedy rows: T = 1
    Te = np.where(T > 0, T, 1.0).astype(np.float64)
    m = x.max(axis=1)
    lse = logsumexp(x.astype(np.float64) / Te[:, None], axis=1)
    qmax = np.exp(m.astype(np.float64) / Te - lse)       # the softmax's largest probability
    feat = svref.est_feature(m, lse.astype(np.float32), T)
    ref = np.clip(logit(qmax), -40, 40)
    assert np.allclose(feat, ref, rtol=0, atol=5e-5 * (1 + np.abs(ref)))
    # saturation: q_max = 1 gives +40, a vanishing q_max gives -40
    sat = svref.est_feature(np.array([0.0, 0.0], np.float32), np.array([0.0, 60.0], np.float32),
                            np.array([1.0, 1.0], np.float32))
    assert sat[0] == 40.0 and sat[1] == -40.0


def _simulate(rng, slope, bias, R, x_scale=2.0, trim=False):
    """R requests of len(bias) drafts: position k survives with probability
    sigmoid(slope * x_k + bias_k) once every earlier one survived."""
    B = len(bias)
    x = rng.normal(0, x_scale, (R, B))
    p = 1 / (1 + np.exp(-(slope * x + np.asarray(bias))))
    survive = rng.random((R, B)) < p
    L = np.where(survive.all(axis=1), B, np.argmin(survive, axis=1)).astype(np.int32)
    w = rng.integers(1, B + 1, R).astype(np.int32) if trim else np.full(R, B, np.int32)
    return x, np.minimum(L, w), w


def test_newton_direction_matches_dense_solve():
    rng = np.random.default_rng(1)
    B = 6
    est = svref.Estimator(B)
    for _ in range(svref.EST_REFIT - 1):
        x, L, w = _simulate(rng, 0.8, [0.5, 0.2, 0.0, -0.3, -0.6, -1.0], 32, trim=True)
        est.observe(x, L, w)
    st = est.st
    H = np.zeros((B + 1, B + 1))
    H[0, 0] = st.h_ss
    H[0, 1:] = H[1:, 0] = st.h_sk[:B]
    H[1:, 1:] = np.diag(st.h_kk[:B])
    g = np.concatenate([[st.g_s], st.g_k[:B]])
    n_s, n_k = st.n_s, np.array(st.n_k[:B])
    delta = np.linalg.solve(H + 1e-3 * np.eye(B + 1), g)
    slope0, bias0 = est.slope, est.bias
    est.observe(np.zeros((0, B)), np.zeros(0, np.int32), np.zeros(0, np.int32))  # the 100th call
    assert est.st.refits == 1 and est.st.calls == 0 and est.st.n_s == 0.0
    assert est.st.last_ds == pytest.approx(delta[0], rel=1e-10)
    step = est.slope - slope0
    assert step == pytest.approx(delta[0] * n_s / (n_s + 50), rel=1e-10)  # no halving needed here
    # with the slope step actually taken, the intercepts' directions solve the
    # remaining rows of the same system
    rest = np.linalg.solve(H[1:, 1:] + 1e-3 * np.eye(B), g[1:] - H[1:, 0] * step)
    assert np.allclose(est.bias - bias0, rest * n_k / (n_k + 50), rtol=1e-10, atol=1e-14)


def test_recovers_the_generating_coefficients():
    rng = np.random.default_rng(2)
    true_s, true_b = 1.0, [1.0, 0.5, 0.0, -0.5, -1.0]
    est = svref.Estimator(5)
    after = []   # coefficients after each of the last 10 refits (each refit fits one batch)
    for c in range(30 * svref.EST_REFIT):
        est.observe(*_simulate(rng, true_s, true_b, 64))
        if c >= 20 * svref.EST_REFIT and est.st.calls == 0:
            after.append((est.slope, est.bias))
    slope = np.mean([a[0] for a in after])
    bias = np.mean([a[1] for a in after], axis=0)
    assert slope == pytest.approx(true_s, abs=0.05)
    assert np.allclose(bias, true_b, atol=0.1)


def test_slope_moves_down_from_above_and_never_turns_negative():
    """From slope 3.0 on drafts generated with slope 1.0 the slope comes down
    near 1 within ten refits (the fix reports 0.96); from the default start on
    drafts without signal it settles near 0 and never goes below it."""
    rng = np.random.default_rng(3)
    est = svref.Estimator(5)
    est.st.slope = 3.0
    seen = []
    for _ in range(10 * svref.EST_REFIT):
        est.observe(*_simulate(rng, 1.0, [1.0, 0.5, 0.0, -0.5, -1.0], 64))
        seen.append(est.slope)
    assert min(seen) >= 0.0 and seen[svref.EST_REFIT - 1] < 3.0
    assert 0.8 <= est.slope <= 1.2
    est = svref.Estimator(5)
    seen = []
    for _ in range(10 * svref.EST_REFIT):
        est.observe(*_simulate(rng, 0.0, [1.0, 0.5, 0.0, -0.5, -1.0], 64))
        seen.append(est.slope)
    assert min(seen) >= 0.0
    assert est.slope <= 0.1


def test_halving_keeps_the_slope_non_negative():
    """A damped slope step larger than the slope is halved until the slope
    stays non-negative; the intercepts still move."""
    rng = np.random.default_rng(4)
    est = svref.Estimator(4)
    est.st.slope = 0.02
    for _ in range(svref.EST_REFIT - 1):
        # strongly negative relation: the full Newton step points far below zero
        est.observe(*_simulate(rng, -2.0, [0.5, 0.0, -0.5, -1.0], 64))
    n_s = est.st.n_s
    s0, b0 = est.slope, est.bias
    est.observe(np.zeros((0, 4)), np.zeros(0, np.int32), np.zeros(0, np.int32))
    full = est.st.last_ds * n_s / (n_s + 50)
    assert s0 + full < 0                                  # the case the rule is about
    step = est.slope - s0
    halved = [full / 2 ** h for h in range(1, 9)]
    ok = [h for h in halved if s0 + h >= 0]
    assert est.slope >= 0.0
    assert step == pytest.approx(ok[0]) if ok else step == 0.0
    assert not np.allclose(est.bias, b0)
