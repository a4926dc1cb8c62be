"""The host planner (workspace layouts, chunk and split counts) built with
g++ under AddressSanitizer and UndefinedBehaviorSanitizer and run over a
sweep of shapes up to the library's limits (tests/host/plan_check.cpp): no
sanitizer report, every layout aligned, in bounds and non-overlapping."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_planner_under_sanitizers():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "plan_check")
        cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
               "-I" + os.path.join(ROOT, "include"),
               "-I" + os.path.join(ROOT, "linear_cross_entropy_tile_amd", "csrc"),
               os.path.join(ROOT, "tests", "host", "plan_check.cpp"), "-o", exe]
        subprocess.run(cmd, check=True, capture_output=True, text=True)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        env.pop("FLCE_D_BUDGET", None)
        env.pop("FLCE_GROUP", None)
        res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        assert res.returncode == 0, res.stdout + res.stderr
        assert "runtime error" not in res.stderr and "ERROR: AddressSanitizer" not in res.stderr
        assert "failures: 0" in res.stdout, res.stdout
