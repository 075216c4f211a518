"""The library from plain C: tests/c_abi/dyadic.c includes include/sscan.h as C11 (gcc),
links libsscan.so and calls the C ABI with caller-owned hipMalloc buffers, no Python in
between.  Without a GPU it runs the validation paths (status codes and messages before
any GPU call); on a GPU the forward and backward of the hand-derived worked example
(A = [-ln 2, -2 ln 2]: every decay a power of 1/2), against its exact values."""
import os
import subprocess

import pytest

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "dyadic")

needs_exe = pytest.mark.skipif(not os.path.exists(EXE), reason="tests/c_abi/dyadic is built by __graft_entry__.build()")


@needs_exe
def test_c_consumer_validation_without_a_gpu():
    r = subprocess.run([EXE, "validate"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "validation ok" in r.stdout


@needs_exe
@pytest.mark.gpu
def test_c_consumer_runs_the_worked_example_on_the_gpu(gpu):
    print("[gpu-case] plain-C consumer: worked example forward + backward", flush=True)
    r = subprocess.run([EXE, "run"], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "worked example ok" in r.stdout
