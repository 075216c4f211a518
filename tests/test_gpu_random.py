"""GPU parity over seeded random problem shapes and launch plans: the forward (with and
without H, either layout where it applies; at DS = 16 also H through the state-group
layout, bitwise the lanes layout's on one pass) and the backward (any lane count and T-chunk
count), and the H-free pair where DS >= 8, against the fp64 oracle; then the same for the
Mamba-style wrapper against its oracle.  Most shapes are small
(the oracle finishes in well under a second each) but cover ragged T and D, single steps
and channels, every DS and both I/O dtypes; a dozen medium ones (up to ~2e7 state updates)
run the same checks with longer sequences and more T-chunks."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import TOL_F32, announce, assert_close, to_dev, tol_for

pytestmark = pytest.mark.gpu

sscan = pytest.importorskip("selective_state_space_sscan_amd")
from selective_state_space_sscan_amd import (Plan, sscan_bwd, sscan_bwd_ckpt, sscan_fwd,  # noqa: E402
                                             sscan_fwd_ckpt, sscan_mamba_bwd, sscan_mamba_fwd)

GR = ["gx", "gdelta", "gb", "gc", "gA", "gh0"]
N_CASES = 48
N_SG = 12  # the last N_SG cases draw only shapes the state-group layout takes, and use it


def draw_case(i, force_sg=None):
    rng = np.random.default_rng(5000 + i)
    B = int(rng.integers(1, 4))
    T = int(rng.choice([1, 2, 31, 32, 33, 63, 64, 65, int(rng.integers(1, 400)), int(rng.integers(400, 1200))]))
    D = int(rng.choice([1, 3, 4, 16, 17, 64, 65, 128, int(rng.integers(1, 160))]))
    DS = int(rng.choice([1, 2, 4, 8, 16]))
    io = "bf16" if rng.random() < 0.3 else "f32"
    h0 = bool(rng.random() < 0.7)
    dhT = bool(rng.random() < 0.6)
    lane_opts = [0] + [l for l in (1, 2, 4, 8, 16) if l <= DS]
    f_lanes = int(rng.choice(lane_opts + ([DS // 2] * 2 if DS >= 4 else [])))
    f_chunks = int(rng.choice([0, 1, 2, 3, 5]))
    sg_ok = DS in (4, 8, 16) and D % 4 == 0 and f_lanes in (0, DS // 2)
    layout = rng.choice([None, "lanes", "state_groups", "state_groups"] if sg_ok else [None, "lanes"])
    b_lanes = int(rng.choice(lane_opts))
    b_chunks = int(rng.choice([0, 1, 2, 4]))
    if force_sg if force_sg is not None else N_CASES - N_SG <= i < N_CASES:
        DS = int(rng.choice([4, 8, 16]))
        D = 4 * int(rng.integers(1, 40))
        f_lanes = int(rng.choice([0, DS // 2]))
        layout = "state_groups"
        b_lanes = int(rng.choice([0] + [l for l in (1, 2, 4, 8, 16) if l <= DS]))
    return B, T, D, DS, io, h0, dhT, (f_lanes, f_chunks, layout), (b_lanes, b_chunks)


def draw_medium_case(i):
    """Shapes up to ~2e7 state updates (a few thousand steps, up to ~1100 channels) with any
    plan, the library's own included."""
    rng = np.random.default_rng(90000 + i)
    B = int(rng.integers(1, 9))
    T = int(rng.integers(1, 5000))
    DS = int(rng.choice([1, 2, 4, 8, 16]))
    D = int(rng.choice([int(rng.integers(1, 1100)), 4 * int(rng.integers(1, 275))]))
    T = max(1, min(T, int(2e7 // (B * D * DS))))
    io = "bf16" if rng.random() < 0.3 else "f32"
    h0 = bool(rng.random() < 0.7)
    dhT = bool(rng.random() < 0.6)
    lane_opts = [0] + [l for l in (1, 2, 4, 8, 16) if l <= DS]
    f_lanes = int(rng.choice(lane_opts + ([DS // 2] * 2 if DS >= 4 else [])))
    f_chunks = int(rng.choice([0, 0, 1, 2, 3, 5, 8, 16]))
    sg_ok = DS in (4, 8, 16) and D % 4 == 0 and f_lanes in (0, DS // 2)
    layout = rng.choice([None, None, "lanes", "state_groups"] if sg_ok else [None, "lanes"])
    b_lanes = int(rng.choice(lane_opts))
    b_chunks = int(rng.choice([0, 0, 1, 2, 4, 8, 16]))
    return B, T, D, DS, io, h0, dhT, (f_lanes, f_chunks, layout), (b_lanes, b_chunks)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_and_plan(gpu, i):
    check_case(gpu, i, draw_case(i))


@pytest.mark.parametrize("i", range(12))
def test_random_medium_shape_and_plan(gpu, i):
    check_case(gpu, 10000 + i, draw_medium_case(i))


def check_case(gpu, i, case):
    B, T, D, DS, io, h0, dhT, fplan, bplan = case
    announce(f"random #{i}: B={B} T={T} D={D} DS={DS} io={io} h0={h0} dhT={dhT} fwd plan={fplan} bwd plan={bplan}")
    w = workloads.custom(B, T, D, DS, io=io, seed=7000 + i, h0_std=0.3 if h0 else 0.0, delta_mu=-1.0,
                         with_dy=True, with_dhT=dhT)
    inp = workloads.make_inputs(w)
    g = to_dev(inp, gpu)
    yr, hTr, Hr = oracle.fwd(inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"], return_H=True)

    # forward without H in the drawn layout, then with H (the lanes layout)
    y, hT = sscan_fwd(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], plan=Plan(*fplan))
    assert_close("y", y, yr, tol_for(io))
    assert_close("hT", hT, hTr, TOL_F32)
    y2, hT2, H = sscan_fwd(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], return_H=True,
                           plan=Plan(fplan[0] if fplan[2] != "state_groups" else 0, fplan[1]))
    assert_close("y (with H)", y2, yr, tol_for(io))
    assert_close("H", H, Hr, TOL_F32)
    if DS == 16 and D % 4 == 0:
        # H through the state-group layout (LDS rows copied out by store waves), whatever
        # the library would pick: its states are the lanes layout's bit for bit on one pass
        fch = fplan[1]
        y3, hT3, H3 = sscan_fwd(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], return_H=True,
                                plan=Plan(0, fch, "state_groups"))
        assert_close("y (state groups, with H)", y3, yr, tol_for(io))
        assert_close("hT (state groups, with H)", hT3, hTr, TOL_F32)
        assert_close("H (state groups)", H3, Hr, TOL_F32)
        if fch == 1:
            _, hT1, H1 = sscan_fwd(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], return_H=True,
                                   plan=Plan(0, 1, "lanes"))
            assert torch.equal(H3, H1) and torch.equal(hT3, hT1)

    ref = oracle.bwd(inp["dy"], inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"], inp["dhT"])
    grads = sscan_bwd(g["dy"], g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], H, g["dhT"], plan=Plan(*bplan))
    for name, a, r in zip(GR, grads, ref):
        assert_close(name, a, r, TOL_F32)

    if DS >= 8:
        # the H-free pair: 8 or 16 lanes per channel in its backward
        _, _, hck = sscan_fwd_ckpt(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"],
                                   plan=Plan(fplan[0] if fplan[2] != "state_groups" else 0, fplan[1]))
        hf_lanes = bplan[0] if bplan[0] >= 8 else 0
        g2 = sscan_bwd_ckpt(g["dy"], g["x"], g["delta"], g["A"], g["b"], g["c"], hck, g["dhT"],
                            plan=Plan(hf_lanes, bplan[1]))
        for name, a, r in zip(GR, g2, ref):
            assert_close(name + " (H-free)", a, r, TOL_F32)


MGR = ["gx", "gdelta_raw", "gb", "gc", "gA_log", "gh0", "gDskip"]
N_MAMBA = 16


@pytest.mark.parametrize("i", range(N_MAMBA))
def test_random_mamba_wrapper(gpu, i):
    B, T, D, DS, io, h0, dhT, fplan, bplan = draw_case(100 + i, force_sg=i % 3 == 0)
    with_D = bool(np.random.default_rng(9000 + i).random() < 0.75)
    announce(f"random mamba #{i}: B={B} T={T} D={D} DS={DS} io={io} h0={h0} dhT={dhT} Dskip={with_D} "
             f"fwd plan={fplan} bwd plan={bplan}")
    w = workloads.custom(B, T, D, DS, io=io, seed=8000 + i, h0_std=0.3 if h0 else 0.0, delta_mu=-1.0,
                         with_dy=True, with_dhT=dhT)
    inp = workloads.make_inputs(w)
    g = to_dev(inp, gpu)
    Dk = g["Dskip"] if with_D else None
    Dr = inp["Dskip"] if with_D else None
    yr, hTr = oracle.mamba_fwd(inp["x"], inp["delta_raw"], inp["A_log"], inp["b"], inp["c"], Dr, inp["h0"])
    gx, gdr, gAl, gb, gc, gD, gh0 = oracle.mamba_bwd(inp["dy"], inp["x"], inp["delta_raw"], inp["A_log"], inp["b"],
                                                     inp["c"], Dr, inp["h0"], inp["dhT"])
    # the gradient for Dskip is formed whether or not the skip term is present
    gD = np.sum(inp["dy"].double().numpy() * inp["x"].double().numpy(), axis=(0, 1))
    ref = [gx, gdr, gb, gc, gAl, gh0, gD]

    y, hT = sscan_mamba_fwd(g["x"], g["delta_raw"], g["A_log"], g["b"], g["c"], Dk, g["h0"], plan=Plan(*fplan))
    assert_close("y", y, yr, tol_for(io))
    assert_close("hT", hT, hTr, TOL_F32)
    hplan = Plan(fplan[0] if fplan[2] != "state_groups" else 0, fplan[1])
    _, _, H = sscan_mamba_fwd(g["x"], g["delta_raw"], g["A_log"], g["b"], g["c"], Dk, g["h0"], return_H=True,
                              plan=hplan)
    grads = sscan_mamba_bwd(g["dy"], g["x"], g["delta_raw"], g["A_log"], g["b"], g["c"], Dk, g["h0"], H, g["dhT"],
                            plan=Plan(*bplan))
    for name, a, r in zip(MGR, grads, ref):
        if name == "gh0" and not h0:
            continue
        assert_close(name, a, r, TOL_F32)

    if DS >= 8:
        _, _, hck = sscan_fwd_ckpt(g["x"], g["delta_raw"], g["A_log"], g["b"], g["c"], g["h0"], mamba=True,
                                   Dskip=Dk, plan=hplan)
        g2 = sscan_bwd_ckpt(g["dy"], g["x"], g["delta_raw"], g["A_log"], g["b"], g["c"], hck, g["dhT"], mamba=True,
                            Dskip=Dk, plan=Plan(bplan[0] if bplan[0] >= 8 else 0, bplan[1]))
        for name, a, r in zip(MGR, g2, ref):
            if name == "gh0" and not h0:
                continue
            assert_close(name + " (H-free)", a, r, TOL_F32)
