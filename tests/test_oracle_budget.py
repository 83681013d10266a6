"""Pins of the oracle's cost-table budget (svref_budget_from_costs).

The planner picks the verify budget b that maximises Theta(b) = tau(b) /
cost[b + R] over every b (TensorRT-LLM PR #17056, description of the
planner: a global argmax over a profiled step-cost table, because the table
is a staircase and Theta need not be unimodal on it; without a profiled
table it does not trim).  tau(b) = R + the b best survivals in rank order.
"""
import numpy as np
import pytest

from oracle import svref

pytestmark = pytest.mark.filterwarnings("ignore")


def brute_force(conf, cost):
    """Theta of every budget from the planner's own windows: tau(b) = R plus
    the survivals of the windows it plans for b, summed request by request."""
    R, B = conf.shape
    th = []
    for b in range(R * B + 1):
        vl, _, surv = svref.plan_windows(conf, b)
        tau = R + sum(float(surv[r, j]) for r in range(R) for j in range(vl[r]))
        th.append(tau / float(cost[b + R]))
    return np.array(th)


def staircase(rng, n_rows, steps):
    """Random non-decreasing step costs over row counts 0..n_rows."""
    edges = np.sort(rng.choice(np.arange(1, n_rows + 1), size=steps, replace=False))
    cost = np.full(n_rows + 1, 1.0)
    for e in edges:
        cost[e:] += rng.uniform(0.05, 0.6)
    return cost.astype(np.float32)


@pytest.mark.parametrize("seed", range(12))
def test_matches_brute_force_over_every_budget(seed):
    rng = np.random.default_rng(seed)
    R, B = int(rng.integers(1, 5)), int(rng.integers(1, 6))
    conf = rng.uniform(0.2, 1.0, (R, B)).astype(np.float32)
    cost = staircase(rng, R * B + R, int(rng.integers(1, R * B + R + 1)))
    b, th = svref.budget_from_costs(conf, cost)
    ref = brute_force(conf, cost)
    order = np.sort(ref)
    if len(order) > 1 and order[-1] - order[-2] < 1e-9 * order[-1]:
        pytest.skip("near tie between two budgets")
    assert b == int(np.argmax(ref))
    assert th == pytest.approx(ref[b], rel=1e-12)


@pytest.mark.parametrize("c,c0,c1,expect", [
    (0.5, 10.0, 1.0, "all"),    # c * c0 = 5 > c1 * R * (1 - c) = 2: Theta increasing
    (0.5, 2.0, 1.0, "none"),    # 1 < 2: Theta decreasing
    (0.25, 40.0, 2.0, "all"),   # 10 > 6
    (0.25, 8.0, 2.0, "none"),   # 2 < 6
])
def test_linear_cost_closed_form(c, c0, c1, expect):
    """B = 1 and equal confidences c: tau(b) = R + b c; with cost c0 + c1 t the
    sign of dTheta/db is that of c c0 - c1 R (1 - c), whatever b, so the
    budget is all or nothing."""
    R = 4
    conf = np.full((R, 1), c, np.float32)
    t = np.arange(R + R + 1, dtype=np.float64)
    cost = (c0 + c1 * t).astype(np.float32)
    b, th = svref.budget_from_costs(conf, cost)
    assert b == (R if expect == "all" else 0)
    assert th == pytest.approx((R + b * c) / (c0 + c1 * (b + R)), rel=1e-7)


def test_global_argmax_not_first_descent():
    """Theta falls after b = 1 and peaks again at b = 8: a descent that stops
    at the first drop would keep 1, the global argmax takes 8."""
    conf = np.full((1, 8), 0.9, np.float32)
    cost = np.array([1.0, 1.0, 1.0, 1.6, 1.6, 1.6, 1.6, 1.65, 1.65, 1.65], np.float32)
    ref = brute_force(conf, cost)
    first_descent = next(b for b in range(len(ref) - 1) if ref[b + 1] < ref[b])
    assert first_descent == 1
    b, th = svref.budget_from_costs(conf, cost)
    assert b == 8
    S = np.cumprod(np.full(8, np.float32(0.9)), dtype=np.float32).astype(np.float64)
    assert th == pytest.approx((1 + S.sum()) / np.float64(np.float32(1.65)), rel=1e-12)


def test_ties_take_the_smaller_budget():
    """Zero survivals after the first draft add nothing to tau: Theta is equal
    for b = 1, 2, 3 under an equal cost, and the smallest wins."""
    conf = np.array([[0.5, 0.0, 0.0, 0.0]], np.float32)
    cost = np.array([1.0, 1.0, 1.0, 1.0, 1.0, 2.0], np.float32)
    b, th = svref.budget_from_costs(conf, cost)
    assert b == 1
    assert th == 1.5


def test_no_table_or_flat_table_does_not_trim():
    rng = np.random.default_rng(5)
    conf = rng.uniform(0.0, 0.05, (6, 4)).astype(np.float32)
    assert svref.budget_from_costs(conf, None)[0] == 24
    flat = np.full(31, 3.0, np.float32)
    flat[:6] = 0.5        # below R rows: outside the range a plan can use
    assert svref.budget_from_costs(conf, flat)[0] == 24


def test_rejects_short_or_invalid_tables():
    conf = np.full((3, 2), 0.5, np.float32)
    with pytest.raises(ValueError):
        svref.budget_from_costs(conf, np.ones(8, np.float32))   # needs 3*2 + 3 + 1 = 10
    bad = np.ones(10, np.float32)
    bad[5] = 0.0
    with pytest.raises(ValueError):
        svref.budget_from_costs(conf, bad)
    bad[5] = np.nan
    with pytest.raises(ValueError):
        svref.budget_from_costs(conf, bad)


def test_budget_is_consistent_with_the_planner():
    """The budget's windows hold exactly its b best survivals: tau from the
    planner's windows equals the oracle's Theta times the cost."""
    rng = np.random.default_rng(9)
    R, B = 32, 6
    conf = (1 / (1 + np.exp(-rng.normal(1, 1.5, (R, B)))) * 0.95 ** np.arange(B)).astype(np.float32)
    cost = staircase(rng, R * B + R, 12)
    b, th = svref.budget_from_costs(conf, cost)
    vl, _, surv = svref.plan_windows(conf, b)
    tau = R + sum(float(surv[r, j]) for r in range(R) for j in range(vl[r]))
    assert vl.sum() == b
    assert tau / float(cost[b + R]) == pytest.approx(th, rel=1e-12)
