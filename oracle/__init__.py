"""fp64 CPU oracle for the selective diagonal state-space scan -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never calls it and
shares no code with it: the arithmetic lives in ``sscan_oracle.c``, a plain
double-precision loop over the definition on the "pssa-100m/pssa_kernels.py"
page (module docstring; forward shape of its scan_fwd, adjoint sweep of its
scan_bwd).

Pins (what fixes the oracle other than itself) are in
``tests/test_oracle_pins.py``: a hand-derived worked example with dyadic
decays, delta = 0, T = 1, DS = 1 and general-DS unrolled sums of products with
exponentials of summed deltas, linearity, chunk composition, the memoryless
limit, central finite differences, autograd of an independent plain loop, and
four exact scaling identities between the gradients.

Inputs may be numpy arrays or CPU torch tensors of any float dtype; they are
converted to float64 (exact for fp32 and bf16).  Outputs are float64 numpy
arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sscan_oracle.c")
_LIB = os.path.join(_HERE, "libsscan_oracle.so")
_lock = threading.Lock()
_lib = None

__all__ = ["build", "fwd", "bwd", "default_threads", "mamba_fwd", "mamba_bwd", "softplus", "softplus_grad"]


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
               "-fno-fast-math", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            # SSCAN_ORACLE_LIBRARY: an instrumented build of sscan_oracle.c (the sanitizer test)
            path = os.environ.get("SSCAN_ORACLE_LIBRARY") or build()
            lib = ctypes.CDLL(path)
            i64, dp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
            lib.sscan_oracle_fwd.argtypes = [i64, i64, i64, i64] + [dp] * 9 + [ci]
            lib.sscan_oracle_fwd.restype = ci
            lib.sscan_oracle_bwd.argtypes = [i64, i64, i64, i64] + [dp] * 14 + [ci]
            lib.sscan_oracle_bwd.restype = ci
            _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _f64(a, shape=None, name="array", required=False):
    if a is None:
        if required:  # a NULL input the C loops would read
            raise ValueError(f"{name} is required")
        return None
    if hasattr(a, "detach"):  # torch tensor
        a = a.detach().to("cpu")
        import torch

        a = a.to(torch.float64).numpy()
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if shape is not None and tuple(a.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(a.shape)}")
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def fwd(x, delta, A, b, c, h0=None, *, return_H=False, nthreads=None):
    """Forward scan in fp64.  Returns (y, hT) or (y, hT, H).

    x, delta: (B,T,D); A: (D,DS); b, c: (B,T,DS); h0: (B,D,DS) or None (zeros).
    """
    x = _f64(x, name="x", required=True)
    B, T, D = x.shape
    A = _f64(A, name="A", required=True)
    DS = A.shape[1]
    delta = _f64(delta, (B, T, D), "delta", required=True)
    A = _f64(A, (D, DS), "A")
    b = _f64(b, (B, T, DS), "b", required=True)
    c = _f64(c, (B, T, DS), "c", required=True)
    h0 = _f64(h0, (B, D, DS), "h0")
    y = np.empty((B, T, D))
    hT = np.empty((B, D, DS))
    H = np.empty((B, T, D, DS)) if return_H else None
    rc = _load().sscan_oracle_fwd(B, T, D, DS, _ptr(x), _ptr(delta), _ptr(A), _ptr(b), _ptr(c), _ptr(h0),
                                  _ptr(y), _ptr(hT), _ptr(H), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"sscan_oracle_fwd failed ({rc})")
    return (y, hT, H) if return_H else (y, hT)


def bwd(dy, x, delta, A, b, c, h0=None, dhT=None, *, nthreads=None):
    """Backward scan in fp64.  Returns (gx, gdelta, gb, gc, gA, gh0).

    gb, gc are summed over channels, gA over batch rows and steps (totals).
    dhT: (B,D,DS) or None (zeros).
    """
    x = _f64(x, name="x", required=True)
    B, T, D = x.shape
    A = _f64(A, name="A", required=True)
    DS = A.shape[1]
    dy = _f64(dy, (B, T, D), "dy", required=True)
    delta = _f64(delta, (B, T, D), "delta", required=True)
    b = _f64(b, (B, T, DS), "b", required=True)
    c = _f64(c, (B, T, DS), "c", required=True)
    h0 = _f64(h0, (B, D, DS), "h0")
    dhT = _f64(dhT, (B, D, DS), "dhT")
    gx = np.empty((B, T, D))
    gdelta = np.empty((B, T, D))
    gb = np.empty((B, T, DS))
    gc = np.empty((B, T, DS))
    gA = np.empty((D, DS))
    gh0 = np.empty((B, D, DS))
    rc = _load().sscan_oracle_bwd(B, T, D, DS, _ptr(dy), _ptr(dhT), _ptr(x), _ptr(delta), _ptr(A), _ptr(b),
                                  _ptr(c), _ptr(h0), _ptr(gx), _ptr(gdelta), _ptr(gb), _ptr(gc), _ptr(gA),
                                  _ptr(gh0), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"sscan_oracle_bwd failed ({rc})")
    return gx, gdelta, gb, gc, gA, gh0


from .mamba import mamba_bwd, mamba_fwd, softplus, softplus_grad  # noqa: E402  (uses fwd/bwd above)
