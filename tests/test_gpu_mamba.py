"""GPU parity of the Mamba-style wrapper (sscan_mamba_fwd / sscan_mamba_bwd) against the
fp64 oracle of oracle/mamba.py on the same seeded inputs: delta = softplus(delta_raw)
(identity above 20), A = -exp(A_log), y = scan + Dskip * x, and the chain-rule gradients.
Tolerances: 1e-4 (fp32 I/O), 2e-2 for y with bf16 I/O; gradients at 1e-4 (the backward
consumes the same bf16 input values as the oracle and keeps fp32 states)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import TOL_F32, announce, assert_close, to_dev, tol_for

pytestmark = pytest.mark.gpu

sscan = pytest.importorskip("selective_state_space_sscan_amd")
from selective_state_space_sscan_amd import Plan, mamba_scan, sscan_mamba_bwd, sscan_mamba_fwd  # noqa: E402

GRADS = ["gx", "gdelta_raw", "gb", "gc", "gA_log", "gh0", "gDskip"]


def mamba_inputs(B, T, D, DS, io, seed, h0=True, dhT=True, big_raw=True):
    w = workloads.custom(B, T, D, DS, io=io, seed=seed, h0_std=0.3 if h0 else 0.0, delta_mu=-1.0,
                         with_dy=True, with_dhT=dhT)
    inp = workloads.make_inputs(w)
    if big_raw and T > 2 and D > 1:
        # a few steps on the identity branch of the softplus (raw > 20): tiny decays there
        raw = inp["delta_raw"].clone()
        raw[0, 1, : min(3, D)] = 21.0
        raw[-1, T - 2, D - 1] = 24.5
        inp["delta_raw"] = raw
    return inp


def oracle_all(inp, with_D=True):
    D = inp["Dskip"] if with_D else None
    y, hT = oracle.mamba_fwd(inp["x"], inp["delta_raw"], inp["A_log"], inp["b"], inp["c"], D, inp["h0"])
    g = oracle.mamba_bwd(inp["dy"], inp["x"], inp["delta_raw"], inp["A_log"], inp["b"], inp["c"], D, inp["h0"],
                         inp["dhT"])
    gx, gdr, gAl, gb, gc, gD, gh0 = g
    return y, hT, (gx, gdr, gb, gc, gAl, gh0, gD)


CASES = [
    # B, T, D, DS, io, h0, dhT, with_D, lanes, chunks (forward), bwd chunks
    (1, 1, 1, 1, "f32", True, True, True, 0, 0, 0),
    (2, 77, 19, 4, "f32", True, True, True, 0, 0, 0),
    (2, 130, 70, 8, "bf16", True, False, True, 0, 0, 0),
    (2, 200, 33, 16, "f32", False, True, True, 0, 0, 0),
    (2, 129, 65, 16, "f32", True, True, False, 16, 1, 1),
    (2, 129, 65, 16, "f32", True, True, True, 8, 3, 2),
    (2, 257, 40, 16, "bf16", True, True, True, 16, 3, 3),
    (1, 300, 300, 16, "f32", True, True, True, 4, 1, 0),
    (3, 64, 300, 2, "f32", True, True, True, 2, 2, 4),
]


@pytest.mark.parametrize("B,T,D,DS,io,h0,dhT,with_D,lanes,fchunks,bchunks", CASES)
def test_mamba_forward_backward(gpu, B, T, D, DS, io, h0, dhT, with_D, lanes, fchunks, bchunks):
    announce(f"mamba B={B} T={T} D={D} DS={DS} io={io} h0={h0} dhT={dhT} D_skip={with_D} "
             f"plan=({lanes},{fchunks}) bwd chunks={bchunks}")
    inp = mamba_inputs(B, T, D, DS, io, seed=500 + B * 7 + T + D + DS, h0=h0, dhT=dhT)
    g = to_dev(inp, gpu)
    Dk = g["Dskip"] if with_D else None
    y, hT, H = sscan_mamba_fwd(g["x"], g["delta_raw"], g["A_log"], g["b"], g["c"], Dk, g["h0"], return_H=True,
                               plan=Plan(lanes, fchunks))
    grads = sscan_mamba_bwd(g["dy"], g["x"], g["delta_raw"], g["A_log"], g["b"], g["c"], Dk, g["h0"], H, g["dhT"],
                            plan=Plan(0, bchunks))
    torch.cuda.synchronize()
    yr, hTr, ref = oracle_all(inp, with_D)
    assert y.dtype == inp["x"].dtype
    assert_close("y", y, yr, tol_for(io))
    assert_close("hT", hT, hTr, TOL_F32)
    for name, a, r in zip(GRADS, grads, ref):
        if name == "gh0" and not h0:
            continue
        if name == "gDskip":
            # the gradient for Dskip is formed whether or not the skip term is present
            r = np.sum(inp["dy"].double().numpy() * inp["x"].double().numpy(), axis=(0, 1))
        assert_close(name, a, r, TOL_F32)


def test_mamba_autograd_matches_oracle(gpu):
    announce("mamba autograd 2x40x48x16 fp32")
    inp = mamba_inputs(2, 40, 48, 16, "f32", seed=611)
    g = to_dev(inp, gpu)
    leaves = {k: g[k].clone().requires_grad_(True) for k in ["x", "delta_raw", "A_log", "b", "c", "Dskip", "h0"]}
    y, hT = mamba_scan(*(leaves[k] for k in ["x", "delta_raw", "A_log", "b", "c", "Dskip", "h0"]))
    L = (y * g["dy"]).sum() + (hT * g["dhT"]).sum()
    L.backward()
    yr, hTr, ref = oracle_all(inp)
    assert_close("y", y.detach(), yr, TOL_F32)
    gx, gdr, gb, gc, gAl, gh0, gD = ref
    for k, r in [("x", gx), ("delta_raw", gdr), ("b", gb), ("c", gc), ("A_log", gAl), ("h0", gh0), ("Dskip", gD)]:
        assert_close("grad " + k, leaves[k].grad, r, TOL_F32)


def test_mamba_workload_size(gpu):
    # the fwd+bwd workload's sizes with the wrapper's inputs (full comparison)
    announce("mamba 8x2048x768x16 fp32 fwd+bwd")
    w = workloads.get("fwd_bwd_f32", with_dhT=True)
    inp = workloads.make_inputs(w)
    g = to_dev(inp, gpu)
    y, hT, H = sscan_mamba_fwd(g["x"], g["delta_raw"], g["A_log"], g["b"], g["c"], g["Dskip"], g["h0"],
                               return_H=True)
    grads = sscan_mamba_bwd(g["dy"], g["x"], g["delta_raw"], g["A_log"], g["b"], g["c"], g["Dskip"], g["h0"], H,
                            g["dhT"])
    torch.cuda.synchronize()
    del H
    yr, hTr, ref = oracle_all(inp)
    assert_close("y", y, yr, TOL_F32)
    assert_close("hT", hT, hTr, TOL_F32)
    for name, a, r in zip(GRADS, grads, ref):
        assert_close(name, a, r, TOL_F32)
