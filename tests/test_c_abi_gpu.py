"""The C ABI from plain C99: tests/c_abi/flce_c_check.c (built by
__graft_entry__.build() with gcc against include/flce.h and the in-tree
library) allocates with the HIP runtime, runs flce_forward and flce_backward
on one stream and checks the zero-weight closed forms, the bounds and the
label-logprob identity with random weights, the invalid-label status word and
host-side argument errors. Run here as a child process."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "flce_c_check")


def test_c_program():
    assert os.path.exists(BIN), f"{BIN} missing: run __graft_entry__.build() first"
    res = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(res.stdout, res.stderr, flush=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "flce_c_check ok" in res.stdout
