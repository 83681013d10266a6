"""Pins of the oracle's near-tie flags: cases built at, and just outside, each
band.

The three decisions of the verify step that jump with their fp inputs are the
ratio test (u against min(1, p(d)/q(d)), Leviathan et al.), the top-p
boundary (the nucleus walk of "Adaptive verification for DFLASH", commit note
on build_speculative_verify_target_probs: top-k/top-p distribution) and the
exponential race that samples the emitted token (Gumbel-max keyed by
position, consolidation study section 2).  The oracle flags a row when the
margin of one of them lies inside its band: |u - ratio| < 1e-5, a kept count
that changes for a top-p target within 1e-6 Z_K of P Z_K, or race keys whose
best two differ by less than 1e-6 (relative).

Each case here is built in closed form with numpy from quantities the pages
or the published algorithms fix (a two-token softmax, the prefix masses of a
sorted row, the race keys w / E), places the margin at 0.5 or 2 times the
band on either side, and checks both the decision and the flag.  The uniforms
come from the oracle's Philox, which its own known-answer pins cover.
"""
import numpy as np
import pytest

SEED = 0x5EED_0001
NEAR_RATIO, NEAR_TOPP, NEAR_RACE, ACCEPT = 4, 8, 16, 1


def _uniforms(oracle, want, lo=0.15, hi=0.85):
    """(rid, pos, u) with acceptance uniforms inside [lo, hi]."""
    out = []
    for rid in range(1000):
        u = oracle.uniform_accept(SEED, rid, 3)
        if lo <= u <= hi:
            out.append((rid, 3, u))
            if len(out) == want:
                return out
    raise AssertionError("not enough uniforms")


# ------------------------------------------------------------------ F1
@pytest.mark.parametrize("frac", [0.5, 2.0])
@pytest.mark.parametrize("side", [+1, -1])
def test_ratio_band(oracle, frac, side):
    """Two-token rows (V = 2, T = 1, no filters): p(0) = 1 / (1 + e^(x1 - x0)).
    q(0) is set so that p(0) / q(0) = u + side * frac * 1e-5.  The draft is
    accepted iff u < ratio, and the row is flagged iff frac < 1."""
    cases = _uniforms(oracle, 6)
    R = len(cases)
    g = np.random.default_rng(7)
    want_ratio = np.array([u + side * frac * 1e-5 for _, _, u in cases])
    x = np.zeros((2 * R, 2), np.float32)
    x[:, 0] = g.uniform(-1.0, 1.0, 2 * R).astype(np.float32)
    t = 0.8 * want_ratio                              # p(0) below the ratio keeps q(0) <= 1
    x[0::2, 0] = np.log(t / (1.0 - t)).astype(np.float32)
    p0 = 1.0 / (1.0 + np.exp(x[:, 1].astype(np.float64) - x[:, 0].astype(np.float64)))
    q = np.zeros((2 * R, 2), np.float32)
    q[0::2, 0] = (p0[0::2] / want_ratio).astype(np.float32)
    q[:, 1] = 1.0 - q[:, 0]
    q[1::2] = 0.5                                    # bonus rows: never read for the test
    drafts = np.zeros(2 * R, np.int32)
    qo = np.arange(R + 1, dtype=np.int32) * 2
    rid = np.array([c[0] for c in cases], np.uint32)
    pos0 = np.array([c[1] for c in cases], np.uint32)
    out = oracle.rejection_sample(x, qo, drafts, q, np.ones(R, np.float32), None, None, rid, pos0,
                                  SEED)
    ratio = p0[0::2] / q[0::2, 0].astype(np.float64)  # the exact ratio of the fp32 q
    u = np.array([c[2] for c in cases])
    assert np.allclose(out["row_ratio"][0::2], ratio, rtol=1e-13, atol=0)
    assert np.array_equal(out["row_u"][0::2], u)
    assert np.all(np.abs(np.abs(u - ratio) - frac * 1e-5) < 0.05e-5)   # the construction holds
    flags = out["row_flags"][0::2]
    assert np.all((flags & ACCEPT > 0) == (side > 0))
    assert np.all((flags & NEAR_RATIO > 0) == (frac < 1.0))


# ------------------------------------------------------------------ F2
def _prefix(x, kc):
    """Prefix masses C_t of the row's order (value desc, id asc) and Z_K, in
    fp64 from the sorted weights exp(x - max), summed left to right."""
    order = np.lexsort((np.arange(x.size), -x.astype(np.float64)))
    w = np.exp(x[order].astype(np.float64) - float(x.max()))[:kc]
    C = np.concatenate([[0.0], np.cumsum(w)])
    return C, C[kc], order


@pytest.mark.parametrize("frac", [0.5, 2.0])
@pytest.mark.parametrize("side", [+1, -1])
@pytest.mark.parametrize("k,t_star", [(0, 2), (0, 5), (4, 2)])
def test_topp_band(oracle, frac, side, k, t_star):
    """P is set so that P Z_K = C_t* + side * frac * 1e-6 Z_K: token t* (in the
    row's order) is kept iff side > 0, and the row is a near tie iff frac < 1,
    with the band of kept counts {t*, t* + 1}."""
    g = np.random.default_rng(100 + t_star + k)
    x = np.sort(g.normal(0, 1.0, 9).astype(np.float32))[::-1].copy()
    g.shuffle(x)
    V = x.size
    kc = k if 0 < k < V else V
    C, zk, order = _prefix(x, kc)
    P = np.float32(C[t_star] / zk + side * frac * 1e-6)
    margin = (float(P) * zk - C[t_star]) / zk            # in units of Z_K
    assert abs(abs(margin) - frac * 1e-6) < 0.1e-6      # fp32 P keeps the construction
    out = oracle.build_target_probs(x[None, :], np.array([0, 1], np.int32),
                                    np.ones(1, np.float32), np.array([k], np.int32),
                                    np.array([P], np.float32), kmax=V)
    n = t_star + 1 if side > 0 else t_star
    assert out["kept_count"][0] == n
    assert np.array_equal(out["kept_idx"][0, :n], order[:n])
    assert np.array_equal(out["order_idx"][0, :kc], order[:kc])
    assert out["row_zk"][0] == pytest.approx(zk, rel=1e-14)
    near = (out["row_flags"][0] & NEAR_TOPP) > 0
    assert near == (frac < 1.0)
    if near:
        assert (out["kept_lo"][0], out["kept_hi"][0]) == (t_star, t_star + 1)
    else:
        assert out["kept_lo"][0] == out["kept_hi"][0] == n


@pytest.mark.parametrize("frac", [0.5, 2.0])
def test_topp_band_is_relative_to_zk(oracle, frac):
    """A row whose Z_K is large (many near-equal logits): the band scales with
    Z_K, so a margin of 2e-6 Z_K (far above 1e-6 in absolute terms) is outside
    it and 0.5e-6 Z_K inside it."""
    g = np.random.default_rng(9)
    x = (3.0 + g.uniform(-0.01, 0.01, 40)).astype(np.float32)
    C, zk, order = _prefix(x, x.size)
    assert zk > 30
    t_star = 17
    P = np.float32(C[t_star] / zk - frac * 1e-6)
    out = oracle.build_target_probs(x[None, :], np.array([0, 1], np.int32),
                                    np.ones(1, np.float32), None, np.array([P], np.float32))
    assert out["kept_count"][0] == t_star
    assert ((out["row_flags"][0] & NEAR_TOPP) > 0) == (frac < 1.0)


def test_topp_band_in_verify_rows(oracle):
    """The verify step carries the same top-p flag on the rows it builds."""
    x = np.array([[2.0, 1.0, 0.5, 0.25, 0.0, -1.0]], np.float32)
    C, zk, _ = _prefix(x[0], 6)
    logits = np.repeat(x, 2, axis=0)
    q = np.full((2, 6), 1 / 6, np.float32)
    for frac, near in ((0.5, True), (2.0, False)):
        P = np.float32(C[3] / zk + frac * 1e-6)
        out = oracle.rejection_sample(logits, np.array([0, 2], np.int32), np.array([0, 0], np.int32),
                                      q, np.ones(1, np.float32), None, np.array([P], np.float32),
                                      None, None, SEED)
        assert ((out["row_flags"][0] & NEAR_TOPP) > 0) == near
        assert out["row_zk"][0] == pytest.approx(zk, rel=1e-14)


# ------------------------------------------------------------------ F3
def _race_uniforms(oracle, rid, pos):
    return np.array([oracle.uniform_race(SEED, rid, pos, 1, v) for v in range(2)])


@pytest.mark.parametrize("frac", [0.5, 2.0])
@pytest.mark.parametrize("side", [+1, -1])
def test_race_band(oracle, frac, side):
    """Bonus-only requests (one row) race over p on V = 2.  The keys are
    p_v / E_v with E_v = -ln U_v; logits are set so that key_0 / key_1 =
    1 + side * frac * 1e-6.  Token 0 wins iff side > 0, and the row is flagged
    iff frac < 1."""
    rids = [r for r in range(400)
            if abs(np.log(np.log(_race_uniforms(oracle, r, 11)[0]) /
                          np.log(_race_uniforms(oracle, r, 11)[1]))) < 1.5][:6]
    R = len(rids)
    x = np.zeros((R, 2), np.float32)
    for a, r in enumerate(rids):
        E = -np.log(_race_uniforms(oracle, r, 11))
        x[a, 0] = np.float32(np.log(E[0] / E[1]) + np.log1p(side * frac * 1e-6))
    # the keys the construction gives, in fp64 from the fp32 logits
    keys = []
    for a, r in enumerate(rids):
        E = -np.log(_race_uniforms(oracle, r, 11))
        w = np.exp(x[a].astype(np.float64) - x[a].max())
        keys.append(w / E)
    keys = np.array(keys)
    rel = (keys[:, 0] - keys[:, 1]) / keys.max(axis=1)
    assert np.all(np.abs(np.abs(rel) - frac * 1e-6) < 0.1e-6)
    q = np.full((R, 2), 0.5, np.float32)
    out = oracle.rejection_sample(x, np.arange(R + 1, dtype=np.int32), np.zeros(R, np.int32), q,
                                  np.ones(R, np.float32), None, None,
                                  np.array(rids, np.uint32), np.full(R, 11, np.uint32), SEED)
    assert np.all(out["next_token"] == (0 if side > 0 else 1))
    assert np.all(((out["row_flags"] & NEAR_RACE) > 0) == (frac < 1.0))


def test_race_band_sees_a_replaced_best(oracle):
    """Three candidates where the race meets a close runner-up before the best
    key (the kept set is visited in the row order, value descending): the
    flag must compare the best against the entry it replaced."""
    hits = 0
    for rid in range(200):
        U = np.array([oracle.uniform_race(SEED, rid, 5, 1, v) for v in range(3)])
        E = -np.log(U)
        # key_1 the best, key_0 a close second (0.5e-6 below), key_2 far below
        x = np.zeros(3, np.float32)
        x[1] = 0.0
        x[0] = np.float32(np.log(E[0] / E[1]) + np.log1p(-0.5e-6))
        x[2] = np.float32(np.log(E[2] / E[1]) - 3.0)
        # the runner-up (token 0) must come first in the row order, so the
        # best replaces it
        if not (0.0 < x[0] < 1.5 and x[2] < x[1] - 1.0):
            continue
        out = oracle.rejection_sample(x[None, :], np.array([0, 1], np.int32),
                                      np.zeros(1, np.int32), np.full((1, 3), 1 / 3, np.float32),
                                      np.ones(1, np.float32), None, None,
                                      np.array([rid], np.uint32), np.array([5], np.uint32), SEED)
        assert out["next_token"][0] == 1
        assert out["row_flags"][0] & NEAR_RACE
        hits += 1
        if hits == 4:
            break
    assert hits == 4
