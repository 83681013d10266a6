"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/pins/svref_sanitize.cpp drives every entry point of oracle/svref.cpp on
small seeded inputs and edge cases; built with g++ and both sanitizers (host
code only, nothing here touches a GPU), any out-of-bounds access, leak or
undefined operation aborts it.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_oracle_runs_clean_under_sanitizers(tmp_path):
    if not shutil.which("g++"):
        pytest.skip("g++ not available")
    exe = tmp_path / "svref_sanitize"
    subprocess.check_call([
        "g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
        "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
        "-I", os.path.join(ROOT, "oracle"),
        os.path.join(ROOT, "oracle", "svref.cpp"),
        os.path.join(ROOT, "tests", "pins", "svref_sanitize.cpp"),
        "-o", str(exe)])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    res = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=600)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]
    assert "ok" in res.stdout
