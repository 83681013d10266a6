"""Pins of the oracle's Philox4x32-10 stream and its uniforms.

Philox4x32-10 is defined by Salmon et al. (SC'11).  The pins are the published
known-answer vectors and rocRAND's engine built from its public header and run
on the host; neither shares code with the oracle.  The conversions to uniforms
are conventions of this library (the pages fix only the seeding granularity,
the keying by position and fp64 acceptance uniforms -- consolidation study,
sections 2-4); they are pinned by range and distribution checks.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

HERE = os.path.dirname(os.path.abspath(__file__))


def _kat():
    rows = []
    with open(os.path.join(HERE, "golden", "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            w = [int(t, 16) for t in line.split()]
            rows.append((w[0:4], w[4:6], w[6:10]))
    return rows


def test_philox_known_answers(oracle):
    kat = _kat()
    assert len(kat) == 3
    for ctr, key, want in kat:
        got = oracle.philox(key, ctr)
        assert [int(x) for x in got] == want


@pytest.fixture(scope="module")
def rocrand_bin(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available for the rocRAND host pin")
    out = tmp_path_factory.mktemp("rocrand") / "rocrand_philox"
    src = os.path.join(HERE, "pins", "rocrand_philox.cpp")
    subprocess.check_call([hipcc, "-O1", "-o", str(out), src], cwd=str(out.parent))
    return str(out)


def test_philox_matches_rocrand_engine(oracle, rocrand_bin):
    g = np.random.default_rng(11)
    words = g.integers(0, 2**32, size=(3000, 6), dtype=np.uint64).astype(np.uint32)
    words[:10] = 0
    words[10:20] = 0xFFFFFFFF
    text = "\n".join(" ".join(f"{int(x):08x}" for x in row) for row in words) + "\n"
    res = subprocess.run([rocrand_bin], input=text, capture_output=True, text=True, check=True)
    lines = res.stdout.strip().split("\n")
    assert len(lines) == len(words)
    for row, line in zip(words, lines):
        key, ctr = row[0:2], row[2:6]
        want = [int(t, 16) for t in line.split()]
        assert [int(x) for x in oracle.philox(key, ctr)] == want


def test_accept_uniform_range_and_distribution(oracle):
    seed = 0x1234_5678_9ABC
    u = np.array([oracle.uniform_accept(seed, r, p) for r in range(200) for p in range(250)])
    assert np.all(u >= 0.0) and np.all(u < 1.0)
    # 53-bit granularity: u * 2^53 is an integer
    assert np.all(np.floor(u * 2.0**53) == u * 2.0**53)
    assert stats.kstest(u, "uniform").pvalue > 1e-3
    # keying: distinct (request, position) pairs give distinct draws
    assert len(np.unique(u)) == len(u)


def test_race_uniform_open_interval_and_distribution(oracle):
    seed = 77
    U = np.array([oracle.uniform_race(seed, 3, 9, 1, v) for v in range(40000)])
    assert np.all(U > 0.0) and np.all(U < 1.0)
    # odd multiples of 2^-24
    k = U * 2.0**24
    assert np.all(k == np.floor(k)) and np.all(k % 2 == 1)
    assert stats.kstest(U, "uniform").pvalue > 1e-3
    # -ln U is Exp(1): the exponential race relies on it
    assert stats.kstest(-np.log(U), "expon").pvalue > 1e-3
    # stream tags separate the verify race from the draft sampler
    U2 = np.array([oracle.uniform_race(seed, 3, 9, 2, v) for v in range(1000)])
    assert not np.array_equal(U[:1000], U2)
