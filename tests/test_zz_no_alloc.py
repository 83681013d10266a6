"""The allocation-free verify entry point (spec_verify_rejection_sample_noalloc)
against the workspace entry point (spec_verify_rejection_sample), through the
C ABI: two calls in a row on the shared static scratch, the second with a
smaller input, each bit-identical to the workspace call and matching the CPU
oracle; sizes beyond the scratch's limits are refused before any launch."""
import ctypes
import os

import numpy as np
import pytest
import torch

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


def _case(seed, R, V, gmax):
    g = np.random.default_rng(seed)
    T = np.where(g.random(R) < 0.2, 0.0, g.uniform(0.5, 1.2, R)).astype(np.float32)
    k = g.choice(np.array([0, 5, 20, 50, 300], np.int32), size=R)
    P = g.choice(np.array([1.0, 0.95, 0.9], np.float32), size=R)
    return W.small_prob_workload(seed, R, g.integers(0, gmax + 1, size=R), V, T=T, k=k, P=P)


def _outs(rows, R):
    return {"accept_len": torch.full((R,), -7, dtype=torch.int32, device="cuda"),
            "out_tokens": torch.full((rows,), -7, dtype=torch.int32, device="cuda"),
            "next_token": torch.full((R,), -7, dtype=torch.int32, device="cuda"),
            "row_flags": torch.full((rows,), 255, dtype=torch.uint8, device="cuda")}


def test_noalloc_matches_the_workspace_entry_point_twice():
    from rejection_sampling_amd import binding as B
    for label, (seed, R, V, gmax) in (("first call", (61, 40, 20007, 9)),
                                      ("second, smaller call", (62, 6, 3001, 3))):
        w = _case(seed, R, V, gmax)
        qo = w.qo_indptr()
        q, d = make_drafts(w, qo, THREADS)
        assert w.num_rows <= B.NOALLOC_MAX_ROWS and R <= B.NOALLOC_MAX_REQUESTS
        progress(f"noalloc {label}: rows={w.num_rows} R={R} V={V}")
        lg, qot, dt, qt = dev_logits(w.logits), dev_i32(qo), dev_i32(d), dev_f32(q)
        prm = params_for(w)
        ref_out = B.rejection_sample(lg, qot, dt, qt, prm)
        out = B.rejection_sample_noalloc(lg, qot, dt, qt, prm, _outs(w.num_rows, R))
        torch.cuda.synchronize()
        for key in ref_out:
            assert torch.equal(ref_out[key].cpu(), out[key].cpu()), f"{label}: {key}"
        got = {k: v.cpu().numpy() for k, v in out.items()}
        compare_verify(got, oracle_verify(w, qo, d, q, threads=THREADS), qo, label=label)


def test_noalloc_refuses_sizes_beyond_its_scratch():
    from rejection_sampling_amd import binding as B
    L = B.load()
    sp = B.Sampling(None, None, None, None, None, 0, B.SV_ALL_GREEDY)
    fake = ctypes.c_void_p(0x10000)   # never dereferenced: the size check comes first
    for rows, R in ((1025, 4), (8, 1025)):
        rc = L.spec_verify_rejection_sample_noalloc(fake, 1, 64, 64, fake, R, rows, fake, None,
                                                    64, None, ctypes.byref(sp), fake, fake, fake,
                                                    None, None)
        assert rc == -2
        assert b"1024" in L.spec_verify_last_error()
