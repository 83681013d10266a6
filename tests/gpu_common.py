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


def params_for(w, all_greedy=False, list_bounded=None) -> B.Params:
    return B.Params(dev_f32(w.temperature), dev_i32(w.top_k), dev_f32(w.top_p),
                    dev_i32(w.request_id), dev_i32(w.position0), w.seed, all_greedy,
                    list_bounded)


def make_drafts(w, qo, threads=None):
    """Draft distributions q (oracle build from the draft logits with each
    request's parameters) and drafted tokens (oracle race over q, stream 2).
    Greedy requests draft argmax(draft logits): their q row is one-hot."""
    q = svref.parallel_draft_probs(w.draft_logits, qo, w.temperature, w.top_k, w.top_p,
                                   w.request_id, w.position0, w.seed, threads)
    d = svref.sample_probs(q, qo, w.request_id, w.position0, w.seed, tag=2)
    return q, d


def oracle_verify(w, qo, drafts, q, verify_cap=None, requests=None, threads=None):
    return svref.parallel_rejection_sample(w.logits, qo, drafts, q, w.temperature, w.top_k,
                                           w.top_p, w.request_id, w.position0, w.seed,
                                           verify_cap=verify_cap, requests=requests,
                                           threads=threads)


def gpu_verify(w, qo, drafts, q, verify_cap=None, all_greedy=False, list_bounded=None):
    lg = dev_logits(w.logits)
    qt = dev_f32(q) if q is not None else None
    out = B.rejection_sample(lg, dev_i32(qo), dev_i32(drafts), qt,
                             params_for(w, all_greedy, list_bounded),
                             dev_i32(verify_cap) if verify_cap is not None else None)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def compare_verify(gpu, ref, qo, requests=None, cap=None, label=""):
    """Check GPU verify outputs against the oracle under the near-tie rules.
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


def compare_build(gpu, ref, flags, qo, T, kmax, label=""):
    """Target-distribution parity: max/argmax exact, lse within 1e-4 absolute,
    kept sets exact on rows without a top-p near tie, probabilities within 1e-5
    relative on those rows."""
    assert np.array_equal(gpu["row_argmax"], ref["row_argmax"]), label
    np.testing.assert_array_equal(gpu["row_max"].astype(np.float64), ref["row_max"])
    np.testing.assert_allclose(gpu["row_lse"], ref["row_lse"], rtol=0, atol=1e-4)
    near = (flags & svref.ROW_NEAR_TOPP) > 0
    ok = ~near
    assert np.array_equal(gpu["kept_count"][ok], ref["kept_count"][ok]), label
    if kmax:
        assert np.array_equal(gpu["kept_idx"][ok], ref["kept_idx"][ok]), label
    if gpu.get("probs") is not None and ref.get("probs") is not None:
        g, rp = gpu["probs"][ok], ref["probs"][ok]
        np.testing.assert_allclose(g, rp, rtol=1e-5, atol=1e-30)
