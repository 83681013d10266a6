"""Pins of the oracle's verify step (accept test, residual, bonus, prefix).

What the pages fix: greedy accepts iff the draft equals the target argmax and
temperature > 0 runs the Leviathan ratio test (consolidation study, section
2); every accept path stops at the planned verify length and the bonus comes
from the last verified row ("Adaptive verification for DFLASH", DFLASH-through-
DSpark commit note); cap-accept verifies the dense window and only trims
acceptance (same page, compact-verify refusal note); trimming changes how many
positions are verified, never the acceptance rule or the output distribution
(TensorRT-LLM PR #17056, description); a uniform ragged layout gives the dense
result and a request's result does not depend on its batch (same pages).

The central pin is the theorem of Leviathan et al. (ICML 2023): the first
emitted token of speculative sampling is distributed exactly as the target p.
It is checked by a chi-square test on 10^6 trials, which fails for a dropped
max(0, .), a wrong ratio direction, a residual that is not renormalised, or a
sample taken from the wrong row.
"""
import numpy as np
import pytest
from scipy import stats
from scipy.special import softmax

from oracle import svref as S
from rejection_sampling_amd.workloads import bf16_bits, bf16_to_f32

V64 = 64


def _chi2_pvalue(counts, p):
    support = p > 0
    assert counts[~support].sum() == 0, "token outside the support was emitted"
    n = counts.sum()
    exp = n * p[support] / p[support].sum()
    chi2 = ((counts[support] - exp) ** 2 / exp).sum()
    return stats.chi2.sf(chi2, support.sum() - 1)


def _trials(oracle, x_rows, d_rows, T, k, P, ntrials, gamma, seed=1234, chunk=250_000):
    """Run `ntrials` single-request verifies with identical rows and request ids
    0..ntrials-1.  Returns (out_tokens [ntrials, gamma+1], accept_len)."""
    rows = gamma + 1
    q1 = oracle.build_target_probs(d_rows, np.array([0, rows], np.int32),
                                   np.array([T], np.float32), np.array([k], np.int32),
                                   np.array([P], np.float32), want_probs=True)["probs"]
    q1 = q1.astype(np.float32)
    outs, lens = [], []
    for c0 in range(0, ntrials, chunk):
        n = min(chunk, ntrials - c0)
        qo = np.arange(n + 1, dtype=np.int32) * rows
        logits = np.ascontiguousarray(np.broadcast_to(x_rows, (n,) + x_rows.shape)
                                      ).reshape(n * rows, -1)
        q = np.ascontiguousarray(np.broadcast_to(q1, (n,) + q1.shape)).reshape(n * rows, -1)
        rid = np.arange(c0, c0 + n, dtype=np.uint32)
        pos0 = np.zeros(n, np.uint32)
        drafts = oracle.sample_probs(q, qo, rid, pos0, seed, tag=2)
        Tn = np.full(n, T, np.float32)
        kn = np.full(n, k, np.int32)
        Pn = np.full(n, P, np.float32)
        res = oracle.parallel_rejection_sample(logits, qo, drafts, q, Tn, kn, Pn, rid, pos0, seed)
        outs.append(res["out_tokens"].reshape(n, rows))
        lens.append(res["accept_len"])
    return np.concatenate(outs), np.concatenate(lens)


def _target(oracle, x_row, T, k, P):
    return oracle.build_target_probs(x_row[None, :], np.array([0, 1], np.int32),
                                     np.array([T], np.float32), np.array([k], np.int32),
                                     np.array([P], np.float32), want_probs=True)["probs"][0]


@pytest.mark.slow
@pytest.mark.parametrize("k,P", [(0, 1.0), (16, 0.9)])
def test_first_emitted_token_follows_target(oracle, k, P):
    g = np.random.default_rng(100 + k)
    x = g.normal(0, 1.5, size=(2, V64)).astype(np.float32)
    d = (x + g.normal(0, 1.0, size=x.shape)).astype(np.float32)
    out, L = _trials(oracle, x, d, 1.0, k, P, 1_000_000, gamma=1)
    p0 = _target(oracle, x[0], 1.0, k, P)
    counts = np.bincount(out[:, 0], minlength=V64)
    assert _chi2_pvalue(counts, p0) > 0.01
    # acceptance is neither always nor never: the residual path is exercised
    assert 0.2 < (L == 1).mean() < 0.95
    # the bonus token after a full accept follows the target of the next row
    p1 = _target(oracle, x[1], 1.0, k, P)
    counts1 = np.bincount(out[L == 1, 1], minlength=V64)
    assert _chi2_pvalue(counts1, p1) > 0.01


@pytest.mark.slow
def test_second_position_conditional_on_first_accept(oracle):
    g = np.random.default_rng(7)
    x = g.normal(0, 1.5, size=(3, V64)).astype(np.float32)
    d = (x + g.normal(0, 0.7, size=x.shape)).astype(np.float32)
    out, L = _trials(oracle, x, d, 1.0, 0, 1.0, 600_000, gamma=2)
    p1 = _target(oracle, x[1], 1.0, 0, 1.0)
    sel = L >= 1
    counts = np.bincount(out[sel, 1], minlength=V64)
    assert _chi2_pvalue(counts, p1) > 0.01


def test_q_equal_p_always_accepts(oracle):
    g = np.random.default_rng(12)
    R, rows = 50, 4
    x = g.normal(0, 2, size=(R * rows, 300)).astype(np.float32)
    qo = np.arange(R + 1, dtype=np.int32) * rows
    T = np.full(R, 0.8, np.float32)
    P = np.full(R, 0.9, np.float32)
    k = np.full(R, 40, np.int32)
    p = oracle.build_target_probs(x, qo, T, k, P, want_probs=True)["probs"].astype(np.float32)
    rid = np.arange(R, dtype=np.uint32)
    pos0 = np.zeros(R, np.uint32)
    drafts = oracle.sample_probs(p, qo, rid, pos0, 5, tag=2)
    res = oracle.rejection_sample(x, qo, drafts, p, T, k, P, rid, pos0, 5)
    # p(d)/q(d) rounds to within 1 ulp of 1; u < 1 - 2^-24 except with tiny odds
    assert np.all(res["accept_len"] == rows - 1)


def test_one_hot_draft_closed_form(oracle):
    """q = one-hot(x0): accept with probability p(x0); after a rejection the
    residual is p without x0, renormalised (Leviathan et al., closed form)."""
    g = np.random.default_rng(13)
    V = 16
    xrow = g.normal(0, 1, size=V).astype(np.float32)
    p = softmax(xrow.astype(np.float64))
    x0 = int(np.argsort(p)[V // 2])
    n = 200_000
    rows = 2
    qo = np.arange(n + 1, dtype=np.int32) * rows
    logits = np.tile(xrow, (n * rows, 1))
    q = np.zeros((n * rows, V), np.float32)
    q[:, x0] = 1.0
    drafts = np.full(n * rows, x0, np.int32)
    rid = np.arange(n, dtype=np.uint32)
    res = oracle.parallel_rejection_sample(logits, qo, drafts, q, np.ones(n, np.float32),
                                           np.zeros(n, np.int32), np.ones(n, np.float32), rid,
                                           np.zeros(n, np.uint32), 99)
    acc = res["accept_len"] == 1
    # accept rate: binomial test against p(x0)
    assert stats.binomtest(int(acc.sum()), n, p[x0]).pvalue > 1e-3
    first = res["out_tokens"].reshape(n, rows)[:, 0]
    rej_tokens = first[~acc]
    assert np.all(rej_tokens != x0)
    resid = p.copy()
    resid[x0] = 0
    counts = np.bincount(rej_tokens, minlength=V)
    assert _chi2_pvalue(counts, resid / resid.sum()) > 0.01


def test_out_of_range_draft_never_accepted(oracle):
    g = np.random.default_rng(14)
    R, rows, V = 30, 5, 200
    x = g.normal(0, 2, size=(R * rows, V)).astype(np.float32)
    qo = np.arange(R + 1, dtype=np.int32) * rows
    q = np.full((R * rows, V), 1.0 / V, np.float32)
    drafts = g.integers(0, V, size=R * rows).astype(np.int32)
    drafts[2::rows] = -1
    drafts[3::rows] = V
    for T in (0.0, 1.0):
        res = oracle.rejection_sample(x, qo, drafts, q, np.full(R, T, np.float32), None, None,
                                      None, None, 3)
        assert np.all(res["accept_len"] <= 2)
        flags = res["row_flags"]
        assert np.all(flags[2::rows] & S.ROW_ACCEPT == 0)
        assert np.all(flags[3::rows] & S.ROW_ACCEPT == 0)


def test_greedy_accept_is_argmax_match(oracle):
    g = np.random.default_rng(15)
    R, rows, V = 40, 5, 300
    x = g.integers(0, 6, size=(R * rows, V)).astype(np.float32)   # ties
    am = np.argmax(x, axis=1)
    drafts = am.copy()
    flip = g.random(R * rows) < 0.3
    drafts[flip] = g.integers(0, V, size=flip.sum())
    qo = np.arange(R + 1, dtype=np.int32) * rows
    res = oracle.rejection_sample(x, qo, drafts, None, np.zeros(R, np.float32))
    for r in range(R):
        s = r * rows
        L = 0
        while L < rows - 1 and drafts[s + L] == am[s + L]:
            L += 1
        assert res["accept_len"][r] == L
        assert np.array_equal(res["out_tokens"][s:s + L], drafts[s:s + L])
        assert res["out_tokens"][s + L] == am[s + L] == res["next_token"][r]
        assert np.all(res["out_tokens"][s + L + 1:s + rows] == -1)


def test_temperature_to_zero_reduces_to_greedy(oracle):
    """T = 1e-6 on rows with a unique max: every non-max weight underflows to
    0 in fp64, so ratio = [d == argmax] and every sample is the argmax."""
    g = np.random.default_rng(16)
    R, rows, V = 60, 5, 500
    # bf16-valued logits: the gap under the max is at least one bf16 step
    # (>= 1/16 near the max), far above T * 745
    x = bf16_to_f32(bf16_bits(g.normal(0, 3, size=(R * rows, V)).astype(np.float32))).copy()
    for r in x:                      # break a tied max by lifting the first one
        if np.sum(r == r.max()) > 1:
            r[np.argmax(r)] += 1.0
    assert all(np.sum(r == r.max()) == 1 for r in x)
    am = np.argmax(x, axis=1)
    drafts = np.where(g.random(R * rows) < 0.6, am, g.integers(0, V, size=R * rows)).astype(
        np.int32)
    qo = np.arange(R + 1, dtype=np.int32) * rows
    q = np.full((R * rows, V), 0.5 / V, np.float32)
    q[np.arange(R * rows), drafts] = 0.5
    cold = oracle.rejection_sample(x, qo, drafts, q, np.full(R, 1e-6, np.float32), None, None,
                                   None, None, 21)
    greedy = oracle.rejection_sample(x, qo, drafts, None, np.zeros(R, np.float32))
    for key in ("accept_len", "out_tokens", "next_token"):
        assert np.array_equal(cold[key], greedy[key]), key


def _ragged_case(seed, R=12, V=400):
    g = np.random.default_rng(seed)
    gam = g.integers(0, 7, size=R).astype(np.int32)
    rows = int((gam + 1).sum())
    qo = np.zeros(R + 1, np.int32)
    np.cumsum(gam + 1, out=qo[1:])
    x = g.normal(0, 2.5, size=(rows, V)).astype(np.float32)
    xd = (x + g.normal(0, 1, size=x.shape)).astype(np.float32)
    T = g.choice([0.0, 0.6, 1.0], size=R).astype(np.float32)
    k = g.choice([0, 5, 30], size=R).astype(np.int32)
    P = g.choice([1.0, 0.8], size=R).astype(np.float32)
    rid = g.integers(0, 1 << 30, size=R).astype(np.uint32)
    pos0 = g.integers(0, 4096, size=R).astype(np.uint32)
    return g, gam, qo, x, xd, T, k, P, rid, pos0


def _drafts(oracle, g, qo, xd, T, k, P, rid, pos0, seed):
    q = oracle.build_target_probs(xd, qo, T, k, P, rid, pos0, seed,
                                  want_probs=True)["probs"].astype(np.float32)
    d = oracle.sample_probs(q, qo, rid, pos0, seed, tag=2)
    return q, d


def test_ragged_layout_equals_single_request_calls(oracle):
    g, gam, qo, x, xd, T, k, P, rid, pos0 = _ragged_case(17)
    seed = 555
    q, d = _drafts(oracle, g, qo, xd, T, k, P, rid, pos0, seed)
    full = oracle.rejection_sample(x, qo, d, q, T, k, P, rid, pos0, seed)
    for r in range(len(gam)):
        s, e = qo[r], qo[r + 1]
        one = oracle.rejection_sample(x[s:e], np.array([0, e - s], np.int32), d[s:e], q[s:e],
                                      T[r:r + 1], k[r:r + 1], P[r:r + 1], rid[r:r + 1],
                                      pos0[r:r + 1], seed)
        assert one["accept_len"][0] == full["accept_len"][r]
        assert one["next_token"][0] == full["next_token"][r]
        assert np.array_equal(one["out_tokens"], full["out_tokens"][s:e])
        assert np.array_equal(one["row_flags"], full["row_flags"][s:e])


def test_batch_permutation_invariance(oracle):
    g, gam, qo, x, xd, T, k, P, rid, pos0 = _ragged_case(18)
    seed = 9
    q, d = _drafts(oracle, g, qo, xd, T, k, P, rid, pos0, seed)
    full = oracle.rejection_sample(x, qo, d, q, T, k, P, rid, pos0, seed)
    perm = g.permutation(len(gam))
    rows_p = np.concatenate([np.arange(qo[r], qo[r + 1]) for r in perm])
    gam_p = gam[perm]
    qo_p = np.zeros_like(qo)
    np.cumsum(gam_p + 1, out=qo_p[1:])
    pm = oracle.rejection_sample(x[rows_p], qo_p, d[rows_p], q[rows_p], T[perm], k[perm],
                                 P[perm], rid[perm], pos0[perm], seed)
    assert np.array_equal(pm["accept_len"], full["accept_len"][perm])
    assert np.array_equal(pm["next_token"], full["next_token"][perm])
    assert np.array_equal(pm["out_tokens"], full["out_tokens"][rows_p])


def test_cap_accept_equals_trimmed_window(oracle):
    """Cap-accept on the dense window == the compact layout whose window is
    trimmed to `cap` drafts (its bonus row is dense row `cap`)."""
    g, gam, qo, x, xd, T, k, P, rid, pos0 = _ragged_case(19)
    seed = 31
    q, d = _drafts(oracle, g, qo, xd, T, k, P, rid, pos0, seed)
    cap = np.array([g.integers(0, gm + 1) for gm in gam], np.int32)
    capped = oracle.rejection_sample(x, qo, d, q, T, k, P, rid, pos0, seed, verify_cap=cap)
    full = oracle.rejection_sample(x, qo, d, q, T, k, P, rid, pos0, seed)
    keep = np.concatenate([np.arange(qo[r], qo[r] + cap[r] + 1) for r in range(len(gam))])
    qo_t = np.zeros_like(qo)
    np.cumsum(cap + 1, out=qo_t[1:])
    trimmed = oracle.rejection_sample(x[keep], qo_t, d[keep], q[keep], T, k, P, rid, pos0, seed)
    assert np.array_equal(capped["accept_len"], trimmed["accept_len"])
    assert np.array_equal(capped["next_token"], trimmed["next_token"])
    assert np.array_equal(capped["accept_len"], np.minimum(full["accept_len"], cap))
    for r in range(len(gam)):
        s = qo[r]
        assert np.array_equal(capped["out_tokens"][s:s + cap[r] + 1],
                              trimmed["out_tokens"][qo_t[r]:qo_t[r + 1]])
        # where the cap does not bind, nothing changes
        if full["accept_len"][r] < cap[r]:
            assert capped["next_token"][r] == full["next_token"][r]


def test_greedy_trim_is_prefix_of_untrimmed(oracle):
    g = np.random.default_rng(20)
    R, rows, V = 30, 8, 256
    x = g.normal(0, 2, size=(R * rows, V)).astype(np.float32)
    am = np.argmax(x, axis=1)
    d = np.where(g.random(R * rows) < 0.8, am, 0).astype(np.int32)
    qo = np.arange(R + 1, dtype=np.int32) * rows
    full = oracle.rejection_sample(x, qo, d, None, np.zeros(R, np.float32))
    for c in range(rows):
        cap = np.full(R, c, np.int32)
        tr = oracle.rejection_sample(x, qo, d, None, np.zeros(R, np.float32), verify_cap=cap)
        assert np.array_equal(tr["accept_len"], np.minimum(full["accept_len"], c))
        for r in range(R):
            L = tr["accept_len"][r]
            s = r * rows
            assert np.array_equal(tr["out_tokens"][s:s + L], full["out_tokens"][s:s + L])


def test_bonus_only_request(oracle):
    """verify_len 0: the request submits only its bonus row and emits a sample
    of the target there."""
    g = np.random.default_rng(21)
    x = g.normal(0, 2, size=(3, 50)).astype(np.float32)
    qo = np.array([0, 1, 3], np.int32)
    q = np.full((3, 50), 0.02, np.float32)
    d = np.array([7, 3, 4], np.int32)
    res = oracle.rejection_sample(x, qo, d, q, np.array([1.0, 1.0], np.float32))
    assert res["accept_len"][0] == 0
    assert res["out_tokens"][0] == res["next_token"][0] >= 0


def test_accept_prefix_bruteforce(oracle):
    g = np.random.default_rng(22)
    for _ in range(20):
        R = int(g.integers(1, 30))
        lens = g.integers(1, 12, size=R)
        qo = np.zeros(R + 1, np.int32)
        np.cumsum(lens, out=qo[1:])
        acc = (g.random(qo[-1]) < 0.75).astype(np.uint8)
        cap = g.integers(-2, 14, size=R).astype(np.int32)
        for vc in (None, cap):
            got = oracle.accept_prefix(acc, qo, vc)
            for r in range(R):
                gamma = lens[r] - 1
                c = gamma if vc is None else max(0, min(int(vc[r]), gamma))
                L = 0
                for j in range(c):
                    if not acc[qo[r] + j]:
                        break
                    L += 1
                assert got[r] == L
