"""The C-ABI library builds, loads without a GPU, exports every symbol the
header declares, and rejects host-detectable misuse with status codes (no
kernel is launched on those paths)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")


@pytest.fixture(scope="module")
def lib():
    from rejection_sampling_amd import binding, build
    if not os.path.exists(binding.LIB_PATH):
        build.build()
    return binding.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_verify_\w+)\s*\(", text)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("spec_verify_build_target_probs", "spec_verify_rejection_sample",
              "spec_verify_plan_windows", "spec_verify_accept_prefix"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_lists_every_export(lib):
    from rejection_sampling_amd import binding
    assert sorted(binding.EXPORTS) == declared_functions()


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.spec_verify_status_string(code)


def test_host_validation_without_gpu(lib):
    """Bad arguments are refused before anything touches the device."""
    from rejection_sampling_amd.binding import Sampling
    sp = Sampling(None, None, None, None, None, 0, 0)
    fake = ctypes.c_void_p(0x10000)   # never dereferenced: validation fails first
    ws = ctypes.c_void_p(0x100000)
    # ld < vocab
    rc = lib.spec_verify_rejection_sample(fake, 1, 10, 20, fake, 1, 2, fake, fake, 20, None,
                                          ctypes.byref(sp), fake, fake, fake, None, ws, 1 << 20,
                                          None)
    assert rc == -2
    # unknown dtype
    rc = lib.spec_verify_rejection_sample(fake, 7, 20, 20, fake, 1, 2, fake, fake, 20, None,
                                          ctypes.byref(sp), fake, fake, fake, None, ws, 1 << 20,
                                          None)
    assert rc == -3
    # draft_probs NULL without the all-greedy hint
    rc = lib.spec_verify_rejection_sample(fake, 1, 20, 20, fake, 1, 2, fake, None, 20, None,
                                          ctypes.byref(sp), fake, fake, fake, None, ws, 1 << 20,
                                          None)
    assert rc == -1
    # workspace too small
    rc = lib.spec_verify_rejection_sample(fake, 1, 20, 20, fake, 1, 2, fake, fake, 20, None,
                                          ctypes.byref(sp), fake, fake, fake, None, ws, 16, None)
    assert rc == -4
    assert b"workspace" in lib.spec_verify_last_error()
    # misaligned bf16 pointer
    rc = lib.spec_verify_rejection_sample(ctypes.c_void_p(0x10001), 1, 20, 20, fake, 1, 2, fake,
                                          fake, 20, None, ctypes.byref(sp), fake, fake, fake,
                                          None, ws, 1 << 20, None)
    assert rc == -3
    # planner: R * block overflow, NULL qo
    rc = lib.spec_verify_plan_windows(fake, 1 << 20, 1 << 20, 1 << 12, 5, fake, fake, None, ws,
                                      1 << 20, None)
    assert rc == -2
    rc = lib.spec_verify_plan_windows(fake, 4, 2, 4, 5, fake, None, None, ws, 1 << 20, None)
    assert rc == -1
    # build: kmax above the list capacity
    rc = lib.spec_verify_build_target_probs(fake, 1, 20, 2, 20, fake, 1, ctypes.byref(sp), None,
                                            0, None, None, None, None, fake, 5000, ws, 1 << 20,
                                            None)
    assert rc == -2
    # empty batches are no-ops
    assert lib.spec_verify_accept_prefix(None, None, 0, None, None, None) == 0
    # acceptance statistics: block above 1024, NULL stats, NULL inputs
    lib.spec_verify_acceptance_stats.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                                 ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    assert lib.spec_verify_acceptance_stats(fake, fake, 4, 1025, fake, None) == -2
    assert lib.spec_verify_acceptance_stats(fake, fake, 4, 16, None, None) == -1
    assert lib.spec_verify_acceptance_stats(None, fake, 4, 16, fake, None) == -1
    # estimator: block outside [1, 64], NULL state
    lib.spec_verify_estimator_init.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    lib.spec_verify_estimator_state_doubles.argtypes = [ctypes.c_int32]
    lib.spec_verify_estimator_state_doubles.restype = ctypes.c_size_t
    assert lib.spec_verify_estimator_init(fake, 0, None) == -2
    assert lib.spec_verify_estimator_init(fake, 65, None) == -2
    assert lib.spec_verify_estimator_init(None, 8, None) == -1
    assert lib.spec_verify_estimator_state_doubles(8) == 6 + 5 * 8
    # cost-table budget: more than 2^20 positions, a table too short, NULL budget,
    # a NULL table with entries, more than 4096 positions without a workspace or
    # with one too small or misaligned
    c = ctypes.c_void_p
    lib.spec_verify_plan_budget.argtypes = [c, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, c,
                                            ctypes.c_int32, c, c, c, ctypes.c_size_t, c]
    assert lib.spec_verify_plan_budget(fake, 1024, 1025, 1024, fake, 1 << 21, fake, None,
                                       None, 0, None) == -2
    assert b"2^20" in lib.spec_verify_last_error()
    assert lib.spec_verify_plan_budget(fake, 4, 3, 4, fake, 15, fake, None, None, 0, None) == -2
    assert b"cost table" in lib.spec_verify_last_error()
    assert lib.spec_verify_plan_budget(fake, 4, 3, 4, fake, 16, None, None, None, 0, None) == -1
    assert lib.spec_verify_plan_budget(fake, 4, 3, 4, None, 16, fake, None, None, 0, None) == -1
    assert lib.spec_verify_plan_budget(fake, 2, 3, 4, fake, 16, fake, None, None, 0, None) == -2
    big = lib.spec_verify_workspace_bytes(0, 1, 65, 64)
    assert lib.spec_verify_plan_budget(fake, 64, 65, 64, fake, 5000, fake, None, None, 0,
                                       None) == -4
    assert lib.spec_verify_plan_budget(fake, 64, 65, 64, fake, 5000, fake, None, fake, big - 1,
                                       None) == -4
    assert lib.spec_verify_plan_budget(fake, 64, 65, 64, fake, 5000, fake, None,
                                       ctypes.c_void_p(0x10008), big, None) == -4
    # layout check: NULL qo_indptr or word, negative sizes
    lib.spec_verify_check_layout.argtypes = [c, ctypes.c_int32, ctypes.c_int32, c, c]
    assert lib.spec_verify_check_layout(None, 3, 9, fake, None) == -1
    assert lib.spec_verify_check_layout(fake, 3, 9, None, None) == -1
    assert lib.spec_verify_check_layout(fake, -1, 9, fake, None) == -2
    # row diagnostics: workspace NULL or too small for the rows; no rows is a no-op
    lib.spec_verify_row_diagnostics.argtypes = [c, ctypes.c_size_t, ctypes.c_int32, c, c, c, c, c]
    assert lib.spec_verify_row_diagnostics(None, 1 << 20, 10, fake, None, None, None, None) == -4
    assert lib.spec_verify_row_diagnostics(ws, 300, 10, fake, None, None, None, None) == -4
    assert lib.spec_verify_row_diagnostics(ws, 300, -1, fake, None, None, None, None) == -2
    assert lib.spec_verify_row_diagnostics(None, 0, 0, None, None, None, None, None) == 0


def test_workspace_query_grows_with_rows(lib):
    a = lib.spec_verify_workspace_bytes(10, 1000, 2, 0)
    b = lib.spec_verify_workspace_bytes(1000, 1000, 2, 0)
    c = lib.spec_verify_workspace_bytes(10, 1000, 256, 16)
    assert 0 < a < b and a < c and a % 256 == 0


def test_sampling_block_layout_matches_header():
    """The binding's ctypes mirror of sv_sampling has the header's fields in
    the header's order."""
    import torch  # noqa: F401  (the binding imports it)
    from rejection_sampling_amd import binding as B
    hdr = open(os.path.join(ROOT, "include", "spec_verify.h")).read()
    body = hdr[hdr.index("typedef struct {", hdr.index("SV_ROW_RESID_EMPTY")):]
    body = re.sub(r"/\*.*?\*/", "", body[: body.index("} sv_sampling;")], flags=re.S)
    names = re.findall(r"(\w+);", body)
    assert names == [f for f, _ in B.Sampling._fields_]


def test_row_order_puts_heavy_requests_first():
    """Host-side row schedule from host values only: a permutation of the rows
    with every row of a heavy request (sampled, top-k off, top-p on; or top-k
    above the single-pass limit) ahead of the others, each group in natural
    order."""
    import numpy as np
    from rejection_sampling_amd import binding as B
    V = 1000
    T = np.array([0.0, 0.8, 1.0, 0.7, 0.9, 1.1], np.float32)
    k = np.array([0, 0, 20, 0, 300, 0], np.int32)
    P = np.array([0.9, 0.9, 0.9, 1.0, 1.0, 0.5], np.float32)
    heavy = [False, True, False, False, True, True]
    qo = np.array([0, 3, 5, 5, 9, 10, 13], np.int32)
    p = B.Params.__new__(B.Params)
    p.host = (T, k, P)
    order = B.heavy_first_order(qo, p, V, device="cpu")
    rows_of = [list(range(int(qo[r]), int(qo[r + 1]))) for r in range(6)]
    first = [i for r in range(6) if heavy[r] for i in rows_of[r]]
    rest = [i for r in range(6) if not heavy[r] for i in rows_of[r]]
    assert order.tolist() == first + rest
    # nothing to reorder when no request (or every request) is heavy
    p.host = (T, np.full(6, 20, np.int32), P)
    assert B.heavy_first_order(qo, p, V, device="cpu") is None
    p.host = (np.ones(6, np.float32), np.zeros(6, np.int32), np.full(6, 0.9, np.float32))
    assert B.heavy_first_order(qo, p, V, device="cpu") is None


def test_sampling_hints_from_host_values():
    """The flags Params.from_host sets come from host values only:
    SV_ALL_GREEDY when no request samples, SV_LIST_BOUNDED when every sampled
    request has 0 < top_k <= 4096."""
    import numpy as np
    from rejection_sampling_amd import binding as B
    T = np.array([0.0, 0.8, 0.5], np.float32)
    assert B.sampling_hints(T, np.array([0, 20, 4096], np.int32)) == (False, True)
    assert B.sampling_hints(T, np.array([0, 20, 0], np.int32)) == (False, False)
    assert B.sampling_hints(T, np.array([5, 20, 4097], np.int32)) == (False, False)
    assert B.sampling_hints(np.zeros(3, np.float32), np.zeros(3, np.int32)) == (True, True)
