"""GPU tests of the C ABI's contract: the device-side layout check (SV_CHECK,
spec_verify_check_layout) and HIP-graph capture of the calls.

Layout check (TensorRT-LLM PR #17056, commit notes on the layout assertions:
refuse rather than degrade silently).  Every invalid qo_indptr used here keeps
its values inside [0, rows + 3] and every per-row buffer holds rows + 3 rows,
so even a kernel that read through the bad layout would stay in bounds; the
check makes the call refuse instead, and the test asserts the refused outputs.

Graph capture (same page, review-pass note: a device-sized host read is a
capture failure).  Each call is captured once into a torch CUDA graph and
replayed on three new input sets copied into the captured tensors, with eager
calls and synchronisations between the replays; every replay must equal the
eager result bit for bit, and the verify outputs must match the oracle.
"""
import os

import numpy as np
import pytest
import torch

from oracle import svref
from rejection_sampling_amd import workloads as W
from tests.gpu_common import (compare_verify, dev_f32, dev_i32, dev_logits, make_drafts,
                              oracle_verify, params_for, progress)

pytestmark = pytest.mark.gpu

THREADS = min(16, os.cpu_count() or 1)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from rejection_sampling_amd import binding
    binding.load()
    yield


def _workload(seed=41, R=8, V=5003):
    g = np.random.default_rng(seed)
    T = np.where(np.arange(R) % 4 == 0, 0.0, g.uniform(0.5, 1.2, R)).astype(np.float32)
    k = np.array([20, 0, 50, 0, 5, 1000, 0, 20], np.int32)[:R]
    P = np.array([0.9, 0.95, 1.0, 1.0, 0.8, 0.9, 0.5, 1.0], np.float32)[:R]
    return W.small_prob_workload(seed, R, g.integers(1, 6, size=R), V, T=T, k=k, P=P)


def _padded(a, extra, fill=0):
    pad = np.full((extra,) + a.shape[1:], fill, a.dtype)
    return np.concatenate([a, pad])


def _verify_with(w, qo, d, q, check, pad=3):
    """Verify call with every per-row buffer padded by `pad` rows."""
    from rejection_sampling_amd import binding as B
    rows = w.num_rows
    R = w.num_requests
    logits = dev_logits(_padded(w.logits, pad))
    qt = dev_f32(_padded(q, pad))
    dt = dev_i32(_padded(np.asarray(d, np.int32), pad))
    prm = params_for(w, check=check)
    out = {"accept_len": torch.full((R,), 77, dtype=torch.int32, device="cuda"),
           "out_tokens": torch.full((rows + pad,), 77, dtype=torch.int32, device="cuda"),
           "next_token": torch.full((R,), 77, dtype=torch.int32, device="cuda"),
           "row_flags": torch.full((rows + pad,), 77, dtype=torch.uint8, device="cuda")}
    # the call itself takes num_rows = rows (the buffers' extra rows are slack)
    call = B.PreparedRejectionSample(logits[:rows], dev_i32(qo), dt[:rows], qt[:rows], prm,
                                     out={k: (v[:rows] if v.numel() == rows + pad else v)
                                          for k, v in out.items()})
    call()
    word = B.workspace_check_word().clone()
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}, int(word.cpu()[0])


def test_check_passes_a_valid_layout_and_changes_nothing():
    w = _workload()
    qo = w.qo_indptr()
    q, d = make_drafts(w, qo, THREADS)
    progress("SV_CHECK on a valid layout")
    plain, _ = _verify_with(w, qo, d, q, check=False)
    checked, word = _verify_with(w, qo, d, q, check=True)
    assert word == 0
    for key in plain:
        assert np.array_equal(plain[key], checked[key]), key
    ref = oracle_verify(w, qo, d, q, threads=THREADS)
    rows = w.num_rows
    compare_verify({k: (v[:rows] if v.size == rows + 3 else v) for k, v in checked.items()}, ref,
                   qo, label="checked")


@pytest.mark.parametrize("case", ["start", "order", "end_short", "end_long"])
def test_check_refuses_a_bad_layout(case):
    from rejection_sampling_amd import binding as B
    w = _workload(seed=43)
    qo = w.qo_indptr().copy()
    q, d = make_drafts(w, qo, THREADS)
    rows = w.num_rows
    if case == "start":
        qo[0] = 1
        want = B.LAYOUT_START
    elif case == "order":
        qo[3] = qo[4] + 2   # qo[3] > qo[4]: decreasing at request 3
        want = B.LAYOUT_ORDER
    elif case == "end_short":
        qo[-1] = rows - 1
        want = B.LAYOUT_END
    else:
        qo[-1] = rows + 3   # inside the padded buffers
        want = B.LAYOUT_END
    assert qo.min() >= 0 and qo.max() <= rows + 3
    progress(f"SV_CHECK refuses layout case={case} qo={qo.tolist()}")
    got, word = _verify_with(w, qo, d, q, check=True)
    assert word & want, (case, word)
    assert np.all(got["accept_len"] == 0)
    assert np.all(got["next_token"] == -1)
    assert np.all(got["out_tokens"][:rows] == -1)
    assert np.all(got["row_flags"][:rows] == 0)
    assert np.all(got["out_tokens"][rows:] == 77)       # nothing written past num_rows
    # the standalone check gives the same word
    w2 = B.check_layout(dev_i32(qo), rows)
    torch.cuda.synchronize()
    assert int(w2.cpu()[0]) == word
    # the build call refuses too
    out = B.build_target_probs(dev_logits(_padded(w.logits, 3))[:rows], dev_i32(qo),
                               params_for(w, check=True), kmax=8)
    torch.cuda.synchronize()
    assert np.all(out["kept_count"].cpu().numpy() == -1)
    assert np.all(out["row_argmax"].cpu().numpy() == -1)
    assert np.all(out["kept_idx"].cpu().numpy() == -1)


def test_check_layout_word_of_valid_planner_output():
    from rejection_sampling_amd import binding as B
    g = np.random.default_rng(5)
    conf = g.random((300, 9)).astype(np.float32)
    vl, qo, _ = B.plan_windows(dev_f32(conf), 1000)
    word = B.check_layout(qo, 1000 + 300)
    torch.cuda.synchronize()
    assert int(word.cpu()[0]) == 0


# ---------------------------------------------------------------- graphs
def test_graph_capture_replays_with_new_data():
    from rejection_sampling_amd import binding as B
    R, V, Bk = 8, 5003, 5
    sets = []
    for s in range(4):
        w = W.small_prob_workload(200 + s, R, Bk, V, T=0.9, k=np.array([0, 20] * 4, np.int32),
                                  P=0.9)
        qo = w.qo_indptr()
        q, d = make_drafts(w, qo, THREADS)
        g = np.random.default_rng(300 + s)
        conf = g.random((R, Bk)).astype(np.float32)
        cost = (1.0 + (np.arange(R * Bk + R + 1) // 7) * 0.3).astype(np.float32)
        acc = (g.random(w.num_rows) < 0.7).astype(np.uint8)
        sets.append((w, qo, q, d, conf, cost, acc))
    w0, qo0, q0, d0, conf0, cost0, acc0 = sets[0]
    # static device inputs (the graph reads these addresses on every replay)
    lg = dev_logits(w0.logits)
    qt = dev_f32(q0)
    dt = dev_i32(d0)
    qot = dev_i32(qo0)
    ct = dev_f32(conf0)
    cst = dev_f32(cost0)
    at = torch.from_numpy(acc0).cuda()
    prm = params_for(w0)
    prm.s.flags &= ~B.SV_LIST_BOUNDED        # keep the split-race launches in the graph
    est = B.AcceptanceEstimator(Bk)
    m = torch.randn(R * Bk, device="cuda") * 3 + 10
    lse = m + torch.rand(R * Bk, device="cuda")

    def calls():
        o = B.rejection_sample(lg, qot, dt, qt, prm)
        vl, qo_p, surv = B.plan_windows(ct, R * Bk // 2)
        bsel, th = B.plan_budget(ct, cst)
        ap = B.accept_prefix(at, qot)
        st = B.acceptance_stats(o["accept_len"], vl, Bk)
        feat, cf = est.predict(m, lse, prm.T)
        est.observe(feat, o["accept_len"], vl)
        return {**{k: v for k, v in o.items()}, "vl": vl, "qo_p": qo_p, "surv": surv,
                "bsel": bsel, "theta": th, "ap": ap, "stats": st, "feat": feat, "conf": cf}

    calls()                                   # eager warm-up sizes the cached workspace
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            static_out = calls()
    torch.cuda.synchronize()
    for rep, (w, qo, q, d, conf, cost, acc) in enumerate(sets[1:] + sets[:1]):
        progress(f"graph replay {rep}")
        lg.copy_(dev_logits(w.logits))
        qt.copy_(dev_f32(q))
        dt.copy_(dev_i32(d))
        qot.copy_(dev_i32(qo))
        ct.copy_(dev_f32(conf))
        cst.copy_(dev_f32(cost))
        at.copy_(torch.from_numpy(acc).cuda())
        state0 = est.state.clone()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        replayed = {k: v.clone() for k, v in static_out.items()}
        state_r = est.state.clone()
        est.state.copy_(state0)               # the eager calls observe from the same state
        eager = calls()                       # eager work between the replays
        torch.cuda.synchronize()
        for k in replayed:
            a, b = replayed[k].cpu(), eager[k].cpu()
            assert torch.equal(a, b), f"replay {rep}: {k} differs from the eager call"
        assert torch.equal(state_r.cpu(), est.state.cpu()), f"replay {rep}: estimator state"
        # the captured call keeps the first set's sampling values (seed,
        # request ids, positions); only the tensors' contents changed
        import dataclasses
        wr = dataclasses.replace(w, temperature=w0.temperature, top_k=w0.top_k, top_p=w0.top_p,
                                 request_id=w0.request_id, position0=w0.position0, seed=w0.seed)
        ref = oracle_verify(wr, qo, d, q, threads=THREADS)
        got = {k: replayed[k].cpu().numpy() for k in ("accept_len", "out_tokens", "next_token",
                                                      "row_flags")}
        compare_verify(got, ref, qo, label=f"graph replay {rep}")
        vl, qo_p, surv = svref.plan_windows(conf, R * Bk // 2)
        assert np.array_equal(replayed["vl"].cpu().numpy(), vl)
        assert np.array_equal(replayed["qo_p"].cpu().numpy(), qo_p)
        b_ref, _ = svref.budget_from_costs(conf, cost)
        assert int(replayed["bsel"].cpu()[0]) == b_ref
        assert np.array_equal(replayed["ap"].cpu().numpy(), svref.accept_prefix(acc, qo))
