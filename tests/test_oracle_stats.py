"""Pins of the oracle's acceptance and trim statistics.

TensorRT-LLM PR #17056, commit note on the trim-regret metric: a request the
planner trimmed (window below the drafted block) that accepted its entire
window was still alive when the cut happened, so the cut cost acceptance; the
trim-regret rate is that group's share of the trimmed requests.  The
consolidation study's section 1 prints per-position acceptance (the share of
drafts whose first j+1 tokens survived), accepted tokens per draft and the
acceptance per drafted token for 3,188 five-token drafts.

Pins: the printed section-1 figures rebuilt from per-draft accepted lengths,
closed forms (no trimming, every trimmed request fully accepted, nothing
accepted), counts read off explicit per-position accept flags on every small
case, invariants, and the clamping of out-of-range device values.
"""
import itertools
import os

import numpy as np

from oracle import svref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "per_position_acceptance.txt")


def _golden():
    vals = {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, *v = line.split()
        vals[k] = [float(x) for x in v]
    return vals


def test_printed_section1_figures():
    """Drafts whose accepted lengths reproduce the printed per-position
    acceptance give back those shares, 1.81 accepted tokens per draft and
    36.2 % per drafted token (within the rounding of the printed percents)."""
    g = _golden()
    surv = g["survival"]
    drafts = int(g["drafts"][0])
    B = len(surv)
    at_least = [round(p * drafts) for p in surv]            # drafts with L > j
    L = np.zeros(drafts, np.int32)
    for j, n in enumerate(at_least):
        L[:n] = j + 1                                       # the first n drafts reach j + 1
    w = np.full(drafts, B, np.int32)
    st = svref.acceptance_stats(L, w, B)
    assert st[0] == drafts and st[1] == 0 and st[2] == 0
    acc = st[5 + B:5 + 2 * B]
    assert np.allclose(acc / drafts, surv, atol=0.5 / drafts)
    assert st[4] == int(g["draft_tokens"][0])               # 15,940 drafted tokens
    assert abs(st[3] - g["accepted_tokens"][0]) <= 0.0005 * drafts * B
    assert abs(st[3] / drafts - g["accepted_per_draft"][0]) < 0.005
    assert abs(st[3] / st[4] - g["acceptance_per_draft_token"][0]) < 0.001


def _flags_count(L, w, B):
    """Counts read off explicit per-position flags: position j of request r is
    offered when the window covers it and accepted when every drafted token up
    to and including it was accepted."""
    R = len(L)
    offered = np.zeros(B, np.int64)
    accepted = np.zeros(B, np.int64)
    trimmed = regret = 0
    for r in range(R):
        wr = min(max(int(w[r]), 0), B)
        lr = min(max(int(L[r]), 0), wr)
        flags = [1] * lr + [0] * (wr - lr)                  # accept flag per verified position
        alive = True
        for j in range(B):
            if j < wr:
                offered[j] += 1
                alive = alive and flags[j] == 1
                if alive:
                    accepted[j] += 1
        if wr < B:
            trimmed += 1
            if all(flags):                                  # never rejected inside the window
                regret += 1
    return trimmed, regret, offered, accepted


def test_every_small_case_matches_explicit_flags():
    for B in (0, 1, 2, 3):
        for R in (1, 2, 3):
            pairs = [(wv, lv) for wv in range(B + 1) for lv in range(wv + 1)]
            for combo in itertools.product(pairs, repeat=R):
                w = np.array([c[0] for c in combo], np.int32)
                L = np.array([c[1] for c in combo], np.int32)
                st = svref.acceptance_stats(L, w, B)
                t, rg, off, acc = _flags_count(L, w, B)
                assert st[0] == R and st[1] == t and st[2] == rg
                assert st[3] == L.sum() and st[4] == w.sum()
                assert np.array_equal(st[5:5 + B], off) and np.array_equal(st[5 + B:], acc)


def test_closed_forms():
    rng = np.random.default_rng(3)
    R, B = 500, 16
    # no trimming: nothing trimmed, no regret, every position offered to all
    w = np.full(R, B, np.int32)
    L = rng.integers(0, B + 1, R).astype(np.int32)
    st = svref.acceptance_stats(L, w, B)
    assert st[1] == 0 and st[2] == 0 and np.all(st[5:5 + B] == R)
    # every request trimmed and fully accepted: all of them are regret
    w = rng.integers(0, B, R).astype(np.int32)
    st = svref.acceptance_stats(w, w, B)
    assert st[1] == R and st[2] == R
    # nothing accepted: only the requests trimmed to an empty window regret
    st = svref.acceptance_stats(np.zeros(R, np.int32), w, B)
    assert st[2] == int((w == 0).sum()) and np.all(st[5 + B:] == 0)


def test_invariants_and_clamping():
    rng = np.random.default_rng(11)
    R, B = 2000, 12
    w = rng.integers(-3, B + 4, R).astype(np.int32)        # out-of-range windows clamp
    L = rng.integers(-3, B + 6, R).astype(np.int32)        # and accepted lengths too
    st = svref.acceptance_stats(L, w, B)
    wc = np.clip(w, 0, B)
    lc = np.minimum(np.clip(L, 0, None), wc)
    off, acc = st[5:5 + B], st[5 + B:]
    assert st[3] == lc.sum() and st[4] == wc.sum()
    assert off.sum() == st[4] and acc.sum() == st[3]        # each position counted once
    assert np.all(acc <= off) and np.all(np.diff(off) <= 0) and np.all(np.diff(acc) <= 0)
    assert st[2] <= st[1] <= st[0] == R
