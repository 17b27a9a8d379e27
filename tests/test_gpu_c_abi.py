"""The C ABI from a C++ program with no Python or torch in its process:
tests/c_abi_check.cpp (built by __graft_entry__.build() into tests/c_abi_check) runs
closed forms through the scan, the fp32 chunked and the bf16 MFMA chunked kernels and
checks the error path, as a child process of the test."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_check")


def test_c_abi_from_cpp():
    # a missing checker is a failure, not a skip: build() compiles it with the library
    assert os.path.exists(EXE), "tests/c_abi_check is not built (run __graft_entry__.build())"
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    print(r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().splitlines()[-1] == "c-abi check ok"
