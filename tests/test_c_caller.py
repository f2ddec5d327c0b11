"""The C ABI from plain C: tests/c_abi_caller.c, built against include/ar.h
and the HIP runtime API only (no Python in the process), must run clean on
the GPU: exact integer sums through one-shot LL, two-shot DIRECT and AUTO,
the error codes, the step end and teardown."""
import os
import subprocess

import pytest

import build_c_caller


def test_c_caller_compiles():
    """Compiling the header and the caller as C11 (CPU only, no GPU needed)."""
    assert os.path.exists(build_c_caller.build())


@pytest.mark.gpu
def test_c_caller_runs():
    exe = build_c_caller.OUT
    assert os.path.exists(exe), "build it first: python tests/build_c_caller.py"
    print("[gpu-test] plain C caller", flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert "c caller ok" in r.stdout
