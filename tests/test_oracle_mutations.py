"""The oracle's pins must catch plausible mistakes.

Each case copies oracle/svref.cpp, plants one mistake by a textual edit,
builds the copy on the CPU and runs the pin tests that should catch it against
that copy (SVREF_LIB).  The case passes when those pins fail.  Nothing here
touches the GPU or the library under test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "svref.cpp")

CASES = [
    ("residual ignores q", "d.p[v] - (double)qrow[v]", "d.p[v]",
     ["test_oracle_verify.py::test_one_hot_draft_closed_form"]),
    ("ratio inverted", "std::min(1.0, pd / q)", "std::min(1.0, q / pd)",
     ["test_oracle_verify.py::test_first_emitted_token_follows_target"]),
    ("sample always from the bonus row", "const int32_t is = s + L;", "const int32_t is = e - 1;",
     ["test_oracle_verify.py::test_greedy_accept_is_argmax_match"]),
    ("top-p drops the boundary token", "if (c < target) { ++n; c += w[t]; }",
     "if (c + w[t] < target) { ++n; c += w[t]; }",
     ["test_oracle_distribution.py::test_topp_is_smallest_set_reaching_p"]),
    ("argmax takes the last tie", "if (x[v] > m) { m = x[v]; a = v; }",
     "if (x[v] >= m) { m = x[v]; a = v; }",
     ["test_oracle_distribution.py::test_greedy_argmax_is_numpy_first_occurrence"]),
    ("top-k keeps one extra", "(prm.k > 0 && prm.k < V) ? prm.k : V",
     "(prm.k > 0 && prm.k < V) ? prm.k + 1 : V",
     ["test_oracle_distribution.py::test_topk_sets_match_lexsort"]),
    ("temperature applied twice", "w[t] = std::exp((x[pi[t]] - m) / prm.T);",
     "w[t] = std::exp((x[pi[t]] - m) / (prm.T * prm.T));",
     ["test_oracle_distribution.py::test_topk_V_topp_1_is_plain_softmax"]),
    ("lse without the max", "out.lse = m / teff + std::log(s);", "out.lse = std::log(s);",
     ["test_oracle_distribution.py::test_lse_matches_scipy"]),
    ("philox round mixes the low half", "uint32_t n0 = hi1 ^ c[1] ^ k[0];",
     "uint32_t n0 = lo1 ^ c[1] ^ k[0];",
     ["test_oracle_philox.py::test_philox_known_answers"]),
    ("acceptance uniform ignores position", "uint32_t ctr[4] = {pos, rid, 0u, 0u};",
     "uint32_t ctr[4] = {0u, rid, 0u, 0u};",
     ["test_oracle_philox.py::test_accept_uniform_range_and_distribution"]),
    ("planner breaks ties by r descending", "return x.r < y.r;", "return x.r > y.r;",
     ["test_oracle_planner.py::test_all_equal_confidence_uses_index_tie_break"]),
    ("survival not cumulative", "acc = (j == 0) ? c : acc * c;", "acc = c;",
     ["test_oracle_planner.py::test_printed_acceptance_is_sum_of_survivals"]),
    ("bonus row not counted in qo_indptr", "qo_indptr[r] + verify_len[r] + 1;",
     "qo_indptr[r] + verify_len[r];",
     ["test_oracle_planner.py::test_rank_allocation_matches_counting"]),
    ("trim regret counts a request one short of its window", "if (trimmed && L == w) stats[2] += 1;",
     "if (trimmed && L + 1 >= w) stats[2] += 1;",
     ["test_oracle_stats.py::test_every_small_case_matches_explicit_flags"]),
    ("per-position acceptance off by one", "if (L > j) stats[5 + block + j] += 1;",
     "if (L >= j) stats[5 + block + j] += 1;",
     ["test_oracle_stats.py::test_printed_section1_figures"]),
    ("estimator labels the first rejected draft accepted", "const double y = k < L ? 1.0 : 0.0;",
     "const double y = 1.0;",
     ["test_oracle_estimator.py::test_recovers_the_generating_coefficients"]),
    ("estimator Schur complement with the wrong sign", "a -= e->h_sk[k] * e->h_sk[k] / d;",
     "a += e->h_sk[k] * e->h_sk[k] / d;",
     ["test_oracle_estimator.py::test_newton_direction_matches_dense_solve"]),
    ("estimator drops a slope step instead of halving it",
     "while (e->slope + step < 0.0 && halvings < 8) {", "while (false) {",
     ["test_oracle_estimator.py::test_halving_keeps_the_slope_non_negative"]),
    ("budget prices the rows without the bonus rows", "const double th = tau / (double)cost[b + R];",
     "const double th = tau / (double)cost[b];",
     ["test_oracle_budget.py::test_linear_cost_closed_form"]),
    ("budget stops at the first descent", "if (th > best) {", "if (th > best && b == best_b + 1) {",
     ["test_oracle_budget.py::test_global_argmax_not_first_descent"]),
    ("budget ties go to the larger budget", "if (th > best) {", "if (th >= best) {",
     ["test_oracle_budget.py::test_ties_take_the_smaller_budget"]),
    ("ratio near-tie band ten times too narrow", "std::fabs(u - ratio) < 1e-5",
     "std::fabs(u - ratio) < 1e-6", ["test_oracle_near_ties.py::test_ratio_band"]),
    ("ratio near-tie flag on one side only", "std::fabs(u - ratio) < 1e-5", "(u - ratio) < 1e-5",
     ["test_oracle_near_ties.py::test_ratio_band"]),
    ("top-p band ten times too wide", "const double band = 1e-6 * zk;",
     "const double band = 1e-5 * zk;", ["test_oracle_near_ties.py::test_topp_band"]),
    ("top-p band absolute instead of relative to Z_K", "const double band = 1e-6 * zk;",
     "const double band = 1e-6;", ["test_oracle_near_ties.py::test_topp_band_is_relative_to_zk"]),
    ("top-p band looks below the target only", "out.n_hi = nucleus_count(w, kc, target + band);",
     "out.n_hi = n;", ["test_oracle_near_ties.py::test_topp_band"]),
    ("top-p flag always set", "out.near_topp = out.n_lo != out.n_hi;", "out.near_topp = true;",
     ["test_oracle_near_ties.py::test_topp_band"]),
    ("race near-tie band ten times too wide", "(best - second) / best < 1e-6",
     "(best - second) / best < 1e-5", ["test_oracle_near_ties.py::test_race_band"]),
    ("race forgets the replaced best", "      second = best;\n      best = key;",
     "      best = key;", ["test_oracle_near_ties.py::test_race_band_sees_a_replaced_best"]),
    ("block test weighs row i with the previous position's weight",
     "A += std::max(p[i] * rows[i].p[x] - q_of(i, x), 0.0);",
     "A += std::max(p[i - 1] * rows[i].p[x] - q_of(i, x), 0.0);",
     ["test_oracle_block.py::test_generated_sequences_follow_the_target",
      "test_oracle_block.py::test_mean_accepted_length_matches_enumeration"]),
    ("block stops at the first failed position", "      tau = i;\n      fl |= SVREF_ROW_ACCEPT;",
     "      if (tau == i - 1) tau = i;\n      fl |= SVREF_ROW_ACCEPT;",
     ["test_oracle_block.py::test_generated_sequences_follow_the_target",
      "test_oracle_block.py::test_mean_accepted_length_matches_enumeration"]),
    ("block residual not reweighted by the block weight",
     "std::max(w * dt.p[v] - q_of(tau, v), 0.0)", "std::max(dt.p[v] - q_of(tau, v), 0.0)",
     ["test_oracle_block.py::test_generated_sequences_follow_the_target"]),
    ("block tests the last position like the others", "    if (i < G) {\n      double A",
     "    if (i <= G) {\n      double A",
     ["test_oracle_block.py::test_generated_sequences_follow_the_target",
      "test_oracle_block.py::test_mean_accepted_length_matches_enumeration"]),
]


@pytest.mark.slow
@pytest.mark.parametrize("name,old,new,pins", CASES, ids=[c[0] for c in CASES])
def test_planted_mistake_is_caught(tmp_path, name, old, new, pins):
    src = open(SRC).read()
    assert src.count(old) == 1, f"pattern for '{name}' not found exactly once"
    mutated = tmp_path / "svref_mut.cpp"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "libsvref_mut.so"
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-shared", "-fPIC",
                           "-I", os.path.join(ROOT, "oracle"), "-o", str(lib), str(mutated)])
    env = dict(os.environ, SVREF_LIB=str(lib))
    ids = [os.path.join(ROOT, "tests", p) for p in pins]
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          *ids], cwd=ROOT, env=env, capture_output=True, text=True)
    assert res.returncode != 0, f"pins did not catch '{name}':\n{res.stdout[-2000:]}"
    assert "failed" in res.stdout
