"""Shared pieces of the GPU parity tests.

Inputs come from rejection_sampling_amd.workloads (raw random pieces) and the
CPU oracle (draft distributions, drafted tokens, expected results); nothing
the GPU computes is ever fed to the oracle or used as an expected value.

Comparison rules (near-tie protocol): unflagged rows must match bit for bit;
a row whose accept decision or emitted token differs must carry the oracle's
near-tie flag that explains it (ratio |u - ratio| < 1e-5, a top-p boundary
within 1e-6 Z_K, or race keys within 1e-6), and such rows must stay under
1e-4 of the rows (at least one allowed only when 1e-4 of the rows is >= 1).
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import svref
from rejection_sampling_amd import binding as B
from rejection_sampling_amd.workloads import BF16, F32


def progress(msg: str) -> None:
    print(f"[case] {msg}", flush=True)


def dev_logits(arr: np.ndarray) -> torch.Tensor:
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr, np.float32)).cuda()


def dev_i32(a) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a.astype(np.int32, copy=False)).cuda()


def dev_f32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def params_for(w, all_greedy=False, list_bounded=None, check=False) -> B.Params:
    """The workload's sampling values uploaded once, with the hints derived on
    the host (Params.from_host); list_bounded overrides that hint."""
    prm = B.Params.from_host(w.temperature, w.top_k, w.top_p, w.request_id, w.position0, w.seed,
                             check=check)
    if all_greedy:
        prm.s.flags |= B.SV_ALL_GREEDY
    if list_bounded is not None:
        prm.s.flags = (prm.s.flags & ~B.SV_LIST_BOUNDED) | (B.SV_LIST_BOUNDED if list_bounded else 0)
    return prm


def make_drafts(w, qo, threads=None):
    """Draft distributions q (oracle build from the draft logits with each
    request's parameters) and drafted tokens (oracle race over q, stream 2).
    Greedy requests draft argmax(draft logits): their q row is one-hot."""
    q = svref.parallel_draft_probs(w.draft_logits, qo, w.temperature, w.top_k, w.top_p,
                                   w.request_id, w.position0, w.seed, threads)
    d = svref.sample_probs(q, qo, w.request_id, w.position0, w.seed, tag=2)
    return q, d


def oracle_verify(w, qo, drafts, q, verify_cap=None, requests=None, threads=None, block=False):
    return svref.parallel_rejection_sample(w.logits, qo, drafts, q, w.temperature, w.top_k,
                                           w.top_p, w.request_id, w.position0, w.seed,
                                           verify_cap=verify_cap, requests=requests,
                                           threads=threads, block=block)


def gpu_verify(w, qo, drafts, q, verify_cap=None, all_greedy=False, list_bounded=None,
               diagnostics=False, block=False):
    """One verify call through the C ABI; with diagnostics, also the per-row
    records (Z_K, Z_N, p(d), mode) the call left in the workspace; block:
    block verification (SV_BLOCK_VERIFY)."""
    lg = dev_logits(w.logits)
    qt = dev_f32(q) if q is not None else None
    prm = params_for(w, all_greedy, list_bounded)
    if block:
        prm.s.flags |= B.SV_BLOCK_VERIFY
    out = B.rejection_sample(lg, dev_i32(qo), dev_i32(drafts), qt, prm,
                             dev_i32(verify_cap) if verify_cap is not None else None)
    res = {k: v for k, v in out.items()}
    if diagnostics:
        res.update({"diag_" + k: v for k, v in B.row_diagnostics(w.num_rows).items()})
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in res.items()}


def compare_verify(gpu, ref, qo, requests=None, cap=None, label="", block=False):
    """Check GPU verify outputs against the oracle under the near-tie rules.
    Under block verification the accepted length is the last position passed,
    so a length mismatch is explained by a near tie at any tested position.
    Returns (number of mismatching requests, flag counts)."""
    qo = np.asarray(qo)
    R = len(qo) - 1
    reqs = range(R) if requests is None else requests
    rows_total = 0
    mism_rows = 0
    flagged = {"ratio": 0, "topp": 0, "race": 0}
    problems = []
    for r in reqs:
        s, e = int(qo[r]), int(qo[r + 1])
        rows_total += e - s
        rf = ref["row_flags"][s:e]
        flagged["ratio"] += int(np.sum(rf & svref.ROW_NEAR_RATIO > 0))
        flagged["topp"] += int(np.sum(rf & svref.ROW_NEAR_TOPP > 0))
        flagged["race"] += int(np.sum(rf & svref.ROW_NEAR_RACE > 0))
        gamma = e - s - 1
        cap_eff = gamma if cap is None else max(0, min(int(cap[r]), gamma))
        ga, ra = int(gpu["accept_len"][r]), int(ref["accept_len"][r])
        same = (ga == ra and int(gpu["next_token"][r]) == int(ref["next_token"][r]) and
                np.array_equal(gpu["out_tokens"][s:e], ref["out_tokens"][s:e]))
        # per-row accept decisions of the tested rows
        gbits = gpu["row_flags"][s:s + cap_eff] & 1
        rbits = ref["row_flags"][s:s + cap_eff] & 1
        bad_rows = np.nonzero(gbits != rbits)[0]
        for jj in bad_rows:
            if not (rf[jj] & (svref.ROW_NEAR_RATIO | svref.ROW_NEAR_TOPP)):
                problems.append(f"request {r} row {jj}: accept bit {gbits[jj]} vs {rbits[jj]} "
                                f"without a near-tie flag")
        if same:
            continue
        mism_rows += 1
        # the first difference must be explained at the deciding position
        j = min(ga, ra)
        expl = False
        if block and ga != ra and np.any(rf[:cap_eff] & (svref.ROW_NEAR_RATIO |
                                                            svref.ROW_NEAR_TOPP)):
            expl = True
        if j < e - s:
            f = rf[j]
            if ga != ra and f & (svref.ROW_NEAR_RATIO | svref.ROW_NEAR_TOPP):
                expl = True
            if ga == ra and f & (svref.ROW_NEAR_RACE | svref.ROW_NEAR_TOPP):
                expl = True
        if not expl:
            problems.append(
                f"request {r}: gpu L={ga} next={gpu['next_token'][r]} out={gpu['out_tokens'][s:e]}"
                f" | ref L={ra} next={ref['next_token'][r]} out={ref['out_tokens'][s:e]}"
                f" flags={rf}")
    assert not problems, f"{label}: unexplained mismatches:\n" + "\n".join(problems[:20])
    budget = max(0, int(1e-4 * rows_total))
    assert mism_rows <= max(budget, 0) or mism_rows == 0, \
        f"{label}: {mism_rows} flagged mismatches over {rows_total} rows exceed 1e-4"
    return mism_rows, flagged


def compare_build(gpu, ref, label=""):
    """Target-distribution parity under the near-tie rules.

    Every row: max and argmax exact, lse within 1e-4 absolute.  Kept sets:
    exact where the oracle's band of kept counts is one count; on a top-p near
    tie (band [kept_lo, kept_hi] of counts for targets within 1e-6 Z_K of
    P Z_K) the GPU's count must lie inside the band.  Either way the GPU's
    kept ids are the first kept_count ids of the oracle's row order.
    Probabilities (rows the oracle gave densely): within 1e-5 relative where
    the counts agree; where a near tie made them differ, proportional to the
    oracle's on the common ids (the same weights over another Z_N).  Returns
    the number of near-tie rows and of those whose counts differ."""
    rows = len(ref["row_argmax"])
    assert np.array_equal(gpu["row_argmax"], ref["row_argmax"]), label
    np.testing.assert_array_equal(gpu["row_max"].astype(np.float64), ref["row_max"])
    np.testing.assert_allclose(gpu["row_lse"], ref["row_lse"], rtol=0, atol=1e-4)
    n_g = gpu["kept_count"]
    lo, hi = ref["kept_lo"], ref["kept_hi"]
    near = lo != hi
    assert np.array_equal(near, (ref["row_flags"] & svref.ROW_NEAR_TOPP) > 0), label
    assert np.array_equal(n_g[~near], ref["kept_count"][~near]), label
    assert np.all((n_g[near] >= lo[near]) & (n_g[near] <= hi[near])), label
    if gpu.get("kept_idx") is not None and ref.get("order_idx") is not None:
        kmax = ref["order_idx"].shape[1]
        t = np.arange(kmax)[None, :]
        upto = np.minimum(n_g, kmax)[:, None]
        want = np.where(t < upto, ref["order_idx"], -1)
        bad = np.nonzero(~np.all(gpu["kept_idx"] == want, axis=1))[0]
        assert bad.size == 0, f"{label}: kept ids differ on rows {bad[:10]}"
    differ = 0
    for i, pr in ref.get("probs_rows", {}).items():
        pg = gpu["probs"][i].astype(np.float64)
        if n_g[i] == ref["kept_count"][i]:
            np.testing.assert_allclose(pg, pr, rtol=1e-5, atol=1e-30, err_msg=f"{label} row {i}")
        else:
            common = (pg > 0) & (pr > 0)
            ratio = pg[common] / pr[common]
            assert np.all(np.abs(ratio / ratio[0] - 1) < 1e-5), f"{label} row {i}"
    differ = int(np.sum(n_g[near] != ref["kept_count"][near]))
    return int(near.sum()), differ


def compare_margins(gpu, ref, qo, drafts, q, label="", zk_tol=5e-7, ratio_tol=5e-6):
    """The GPU's decision quantities against the oracle's on every sampled row
    both built: Z_K relative error below zk_tol (half the 1e-6 Z_K top-p band)
    and ratio error below ratio_tol (half the 1e-5 ratio band) on tested
    drafts, so an unflagged decision cannot differ.  Returns the maximum
    errors."""
    zk_r = ref["row_zk"]
    mode = gpu["diag_mode"]
    built = ~np.isnan(zk_r) & (mode >= 2)
    rel = np.abs(gpu["diag_zk"][built] / zk_r[built] - 1.0)
    zk_err = float(rel.max()) if rel.size else 0.0
    assert zk_err < zk_tol, f"{label}: max |Z_K gpu / Z_K ref - 1| = {zk_err:.3g}"
    tested = ~np.isnan(ref["row_ratio"]) & (mode >= 2)
    idx = np.nonzero(tested)[0]
    d = np.asarray(drafts)[idx]
    qd = q[idx, d].astype(np.float64)
    pd = gpu["diag_pd"][idx]
    ratio_g = np.where(qd > 0, np.minimum(1.0, pd / np.where(qd > 0, qd, 1.0)),
                       np.where(pd > 0, 1.0, 0.0))
    err = np.abs(ratio_g - ref["row_ratio"][idx])
    ratio_err = float(err.max()) if err.size else 0.0
    assert ratio_err < ratio_tol, f"{label}: max |ratio gpu - ratio ref| = {ratio_err:.3g}"
    return zk_err, ratio_err, int(built.sum()), int(idx.size)
