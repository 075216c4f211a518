"""fp64 oracle for the Mamba-style wrapper around the scan -- TEST INFRASTRUCTURE.

The POPCORNBENCH page builds its module around the same recurrence: the step size
is the softplus of a projection output, the decay rates come from a learned log
parameter, and the output gets a per-channel skip term.  In that page's notation
(steps 1, 4 and 9 of its forward, and its numerically stable softplus, which
returns its argument above 20):

    delta = softplus(delta_raw)          softplus(r) = r if r > 20 else log(1 + e^r)
    A     = -exp(A_log)
    y     = scan(x, delta, A, b, c, h0) + Dskip * x

The scan itself is this package's fp64 oracle (``oracle.fwd`` / ``oracle.bwd``).
The backward is the chain rule through the three maps:

    d delta / d delta_raw = 1 if r > 20 else e^r / (1 + e^r)
    d A / d A_log         = -exp(A_log) = A
    gx += dy * Dskip,     gDskip[d] = sum over b, t of dy * x

Everything is evaluated in float64 numpy; pins are in
``tests/test_oracle_mamba_pins.py``.
"""
from __future__ import annotations

import numpy as np

from . import _f64, bwd, fwd

SOFTPLUS_THRESHOLD = 20.0


def softplus(raw):
    """Thresholded softplus in fp64 (the POPCORNBENCH page's stable form)."""
    r = _f64(raw, name="delta_raw")
    small = np.minimum(r, SOFTPLUS_THRESHOLD)  # keeps exp() finite on the branch not taken
    return np.where(r > SOFTPLUS_THRESHOLD, r, np.log1p(np.exp(small)))


def softplus_grad(raw):
    """Derivative of the thresholded softplus: 1 above the threshold, else the logistic."""
    r = _f64(raw, name="delta_raw")
    small = np.minimum(r, SOFTPLUS_THRESHOLD)
    logistic = np.exp(small) / (1.0 + np.exp(small))
    return np.where(r > SOFTPLUS_THRESHOLD, 1.0, logistic)


def decay_rates(A_log):
    """A = -exp(A_log), in fp64."""
    return -np.exp(_f64(A_log, name="A_log"))


def mamba_fwd(x, delta_raw, A_log, b, c, Dskip=None, h0=None, *, return_H=False, nthreads=None):
    """Returns (y, hT) or (y, hT, H) of the wrapped scan; Dskip (D,) or None (no skip)."""
    x64 = _f64(x, name="x")
    out = fwd(x64, softplus(delta_raw), decay_rates(A_log), b, c, h0, return_H=return_H, nthreads=nthreads)
    y = out[0]
    if Dskip is not None:
        y = y + _f64(Dskip, (x64.shape[2],), "Dskip")[None, None, :] * x64
    return (y,) + tuple(out[1:])


def mamba_bwd(dy, x, delta_raw, A_log, b, c, Dskip=None, h0=None, dhT=None, *, nthreads=None):
    """Gradients of sum(dy*y) + sum(dhT*hT) for mamba_fwd.

    Returns (gx, gdelta_raw, gA_log, gb, gc, gDskip, gh0); gDskip is None without Dskip.
    """
    x64 = _f64(x, name="x")
    dy64 = _f64(dy, x64.shape, "dy")
    A = decay_rates(A_log)
    gx, gdelta, gb, gc, gA, gh0 = bwd(dy64, x64, softplus(delta_raw), A, b, c, h0, dhT, nthreads=nthreads)
    gdelta_raw = gdelta * softplus_grad(delta_raw)
    gA_log = gA * A
    gD = None
    if Dskip is not None:
        D = _f64(Dskip, (x64.shape[2],), "Dskip")
        gx = gx + dy64 * D[None, None, :]
        gD = np.sum(dy64 * x64, axis=(0, 1))
    return gx, gdelta_raw, gA_log, gb, gc, gD, gh0
