"""Helpers shared by the GPU parity tests: move seeded inputs to the device,
compare GPU outputs with the fp64 oracle (max|err| / max|ref| per tensor, the
metric of the pssa_kernels.py page's selftest)."""
import sys

import numpy as np
import torch


TOL_F32 = 1e-4   # max relative error for fp32 I/O
TOL_BF16 = 2e-2  # max relative error for bf16 I/O (fp32 state)


def tol_for(io: str) -> float:
    return TOL_F32 if io == "f32" else TOL_BF16


def announce(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(inp, dev):
    return {k: (None if v is None else v.to(dev)) for k, v in inp.items()}


def f64(t):
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu", torch.float64).numpy()


def rel_err(a, ref) -> float:
    a = f64(a)
    ref = f64(ref)
    if ref.size == 0:
        return 0.0
    den = float(np.max(np.abs(ref)))
    num = float(np.max(np.abs(a - ref)))
    return num / den if den > 0 else num


def assert_close(name, a, ref, tol):
    e = rel_err(a, ref)
    assert e < tol, f"{name}: max rel err {e:.3e} >= {tol:.1e}"
    return e
