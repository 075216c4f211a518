"""Helpers shared by the GPU parity tests: move seeded inputs to the device,
compare GPU outputs with the fp64 oracle (max|err| / max|ref| per tensor, the
metric of the pssa_kernels.py page's selftest), and sample rows at full size."""
import sys

import numpy as np
import torch

import oracle

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


def sample_rows(B, D, n, seed=1234):
    """(b, d) rows to check at full size: the corners plus seeded random picks."""
    rng = np.random.default_rng(seed)
    rows = {(0, 0), (B - 1, D - 1), (0, D - 1), (B - 1, 0)}
    while len(rows) < min(n, B * D):
        rows.add((int(rng.integers(B)), int(rng.integers(D))))
    return sorted(rows)


def oracle_rows(inp, rows, T0=0, T1=None):
    """fp64 oracle on single (b, d) rows over steps [T0, T1): returns {row: (y (T,), hT (DS,))}."""
    out = {}
    x, dl, A, b, c, h0 = (inp[k] for k in ("x", "delta", "A", "b", "c", "h0"))
    T1 = x.shape[1] if T1 is None else T1
    for (bb, d) in rows:
        xr = x[bb:bb + 1, T0:T1, d:d + 1]
        dr = dl[bb:bb + 1, T0:T1, d:d + 1]
        hr = None if h0 is None else h0[bb:bb + 1, d:d + 1]
        y, hT = oracle.fwd(xr, dr, A[d:d + 1], b[bb:bb + 1, T0:T1], c[bb:bb + 1, T0:T1], hr, nthreads=1)
        out[(bb, d)] = (y[0, :, 0], hT[0, 0])
    return out
