"""The C ABI without Python: tests/capi/capi_check (built by
__graft_entry__.build()) allocates device memory with hipMalloc, calls the
fp16 and bf16 GEMM and both GEMV layouts through include/sdt.h, checks every
product against the CPU oracle's C entry points, and checks the error
statuses.  Run as a child process."""
import os
import subprocess

import pytest

from gpu_helpers import say

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "capi", "capi_check")


def test_c_abi_program():
    assert os.path.exists(BIN), f"{BIN} is not built: run __graft_entry__.build()"
    say("C ABI program tests/capi/capi_check")
    res = subprocess.run([BIN], capture_output=True, text=True, timeout=100)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "CAPI OK" in res.stdout, out[-4000:]
