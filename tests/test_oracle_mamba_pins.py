"""Pins for the fp64 oracle of the Mamba-style wrapper (oracle/mamba.py): values fixed
by the POPCORNBENCH page's definition and by mathematics, not by re-running the
oracle's own chain rule.

Wrapper (POPCORNBENCH page, steps 1, 4 and 9 of the module's forward, and its stable
softplus that returns its argument above 20):
    delta = softplus(delta_raw),  A = -exp(A_log),  y = scan(x, delta, A, b, c, h0) + Dskip * x
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from test_oracle_pins import DYADIC, rel_err

LN2 = math.log(2.0)


def case(B, T, D, DS, seed, dhT=True):
    w = workloads.custom(B, T, D, DS, seed=seed, delta_mu=-1.0, h0_std=0.3, with_dy=True, with_dhT=dhT)
    inp = workloads.make_inputs(w)
    return {k: (None if v is None else v.double().numpy()) for k, v in inp.items()}


def test_softplus_values():
    r = np.array([0.0, 25.0, 20.5, -40.0, 1.0, -1.0])
    got = oracle.softplus(r)
    assert got[0] == pytest.approx(LN2, rel=1e-15)          # log 2
    assert got[1] == 25.0 and got[2] == 20.5                # the identity branch above 20
    assert got[3] == pytest.approx(math.exp(-40.0), rel=1e-12)  # log(1 + e^r) ~ e^r far below 0
    assert got[4] == pytest.approx(math.log(1.0 + math.e), rel=1e-15)
    assert got[4] - got[5] == pytest.approx(1.0, rel=1e-15)  # softplus(r) - softplus(-r) = r
    # at the threshold itself the log branch is taken, within e^-20 of the identity
    assert 0 < oracle.softplus(np.array([20.0]))[0] - 20.0 < 2.1e-9


def test_softplus_derivative_values():
    g = oracle.softplus_grad(np.array([0.0, 25.0, -40.0, 3.0, -3.0]))
    assert g[0] == 0.5 and g[1] == 1.0
    assert g[2] == pytest.approx(math.exp(-40.0), rel=1e-12)
    assert g[3] + g[4] == pytest.approx(1.0, rel=1e-15)  # logistic(r) + logistic(-r) = 1


def test_skip_term_alone():
    # with b = 0 and h0 = 0 the state stays 0 whatever delta and A are: y = Dskip * x exactly
    e = case(2, 9, 5, 4, seed=31)
    b0 = np.zeros_like(e["b"])
    y, hT = oracle.mamba_fwd(e["x"], e["delta_raw"], e["A_log"], b0, e["c"], e["Dskip"], None)
    assert np.array_equal(y, e["Dskip"][None, None, :] * e["x"])
    assert np.array_equal(hT, np.zeros_like(hT))


def test_dyadic_example_through_the_wrapper():
    # A = -exp(A_log) with A_log = log(ln 2), log(2 ln 2) gives A = [-ln 2, -2 ln 2] of the
    # hand-derived example; delta_raw = log(e^delta - 1) inverts the softplus; Dskip = 0.5
    v = {k: np.array(val, dtype=np.float64) for k, val in DYADIC.items()}
    A_log = np.log(-v["A"])
    raw = np.log(np.expm1(v["delta"]))
    D = np.full(v["x"].shape[2], 0.5)
    y, hT = oracle.mamba_fwd(v["x"], raw, A_log, v["b"], v["c"], D, v["h0"])
    yexp = np.array([6.0, 1.0625, -10.9375]).reshape(1, 3, 1) + 0.5 * v["x"]
    assert rel_err(y, yexp) < 1e-14
    assert rel_err(hT, np.array([12.0, 0.53125]).reshape(1, 1, 2)) < 1e-14


def _loss(e, **over):
    v = dict(e)
    v.update(over)
    y, hT = oracle.mamba_fwd(v["x"], v["delta_raw"], v["A_log"], v["b"], v["c"], v["Dskip"], v["h0"], nthreads=1)
    return float(np.sum(e["dy"] * y) + np.sum(e["dhT"] * hT))


def test_gradients_match_finite_differences():
    e = case(2, 6, 3, 4, seed=32)
    e["delta_raw"][0, 1, 2] = 23.0  # one step on the identity branch of the softplus
    got = oracle.mamba_bwd(e["dy"], e["x"], e["delta_raw"], e["A_log"], e["b"], e["c"], e["Dskip"], e["h0"],
                           e["dhT"])
    names = {"x": 0, "delta_raw": 1, "A_log": 2, "b": 3, "c": 4, "Dskip": 5, "h0": 6}
    eps = 1e-6
    for nm, k in names.items():
        base = e[nm]
        fd = np.zeros_like(base)
        it = np.nditer(base, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            p = base.copy()
            m = base.copy()
            p[idx] += eps
            m[idx] -= eps
            fd[idx] = (_loss(e, **{nm: p}) - _loss(e, **{nm: m})) / (2 * eps)
        assert rel_err(got[k], fd) < 1e-7, nm


def _torch_wrapper_loop(x, raw, A_log, b, c, Dskip, h0):
    # the pssa_kernels.py page's scan_reference loop transcribed into torch fp64, with the
    # wrapper's maps around it (torch's own softplus with threshold 20); a pin because the
    # pages print it, its gradients from autograd
    delta = torch.nn.functional.softplus(raw, beta=1.0, threshold=20.0)
    A = -torch.exp(A_log)
    h = h0
    ys = []
    for t in range(x.shape[1]):
        h = torch.exp(delta[:, t, :, None] * A) * h + delta[:, t, :, None] * b[:, t, None, :] * x[:, t, :, None]
        ys.append((h * c[:, t, None, :]).sum(-1))
    return torch.stack(ys, 1) + Dskip * x, h


@pytest.mark.parametrize("shape", [(2, 7, 64, 16), (1, 20, 5, 4)])
def test_gradients_match_autograd_of_plain_loop(shape):
    B, T, D, DS = shape
    e = case(B, T, D, DS, seed=33 + T)
    e["delta_raw"][0, 0, :3] = 21.0  # identity branch
    keys = ["x", "delta_raw", "A_log", "b", "c", "Dskip", "h0"]
    ts = {k: torch.tensor(e[k], dtype=torch.float64, requires_grad=True) for k in keys}
    y, hT = _torch_wrapper_loop(*(ts[k] for k in keys))
    L = (torch.tensor(e["dy"]) * y).sum() + (torch.tensor(e["dhT"]) * hT).sum()
    ref = torch.autograd.grad(L, [ts[k] for k in keys])
    got = oracle.mamba_bwd(e["dy"], e["x"], e["delta_raw"], e["A_log"], e["b"], e["c"], e["Dskip"], e["h0"], e["dhT"])
    for nm, g, r in zip(keys, got, ref):
        assert rel_err(g, r.numpy()) < 1e-12, nm
    yo, hTo = oracle.mamba_fwd(e["x"], e["delta_raw"], e["A_log"], e["b"], e["c"], e["Dskip"], e["h0"])
    assert rel_err(yo, y.detach().numpy()) < 1e-12 and rel_err(hTo, hT.detach().numpy()) < 1e-12


def test_no_skip_means_plain_scan_of_the_transformed_inputs():
    e = case(1, 11, 6, 8, seed=34)
    y, hT = oracle.mamba_fwd(e["x"], e["delta_raw"], e["A_log"], e["b"], e["c"], None, e["h0"])
    # the generator's delta is torch's fp32 softplus of the same raw draw and its A_log is
    # log(-A) in fp32, so the plain scan on (delta, A) agrees to fp32 rounding of the inputs
    y2, hT2 = oracle.fwd(e["x"], e["delta"], e["A"], e["b"], e["c"], e["h0"])
    assert rel_err(y, y2) < 1e-5 and rel_err(hT, hT2) < 1e-5
    g = oracle.mamba_bwd(e["dy"], e["x"], e["delta_raw"], e["A_log"], e["b"], e["c"], None, e["h0"], e["dhT"])
    assert g[5] is None
