"""GPU edge cases of the scan fixed by mathematics rather than by the oracle alone:

* the hand-derived dyadic worked example (every decay a power of 1/2), forward and all
  six gradients, in every lane layout;
* the memoryless limit (A = -1e6: every decay underflows to exactly 0, so
  h_t = delta_t b_t x_t and y_t = delta_t x_t <b_t, c_t>), the caveat the POPCORNBENCH
  page raises about exp(delta A) underflowing;
* the wrapper's softplus far below zero (delta_raw = -40: softplus(r) = log(1 + e^r),
  which is e^r to within e^(2r)/2), POPCORNBENCH page, its stable softplus;
* inputs broadcast over the batch dimension (expanded b, c and x).

Tolerances as elsewhere: max|err| / max|ref| per tensor, 1e-4 for fp32 I/O."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import TOL_F32, announce, assert_close, f64, to_dev
from test_oracle_pins import DYADIC, LN2

pytestmark = pytest.mark.gpu

sscan = pytest.importorskip("selective_state_space_sscan_amd")
from selective_state_space_sscan_amd import (Plan, sscan_bwd, sscan_fwd, sscan_mamba_bwd,  # noqa: E402
                                             sscan_mamba_fwd)

GRADS = ["gx", "gdelta", "gb", "gc", "gA", "gh0"]

# the hand-derived values of the dyadic example (derivation beside DYADIC in the oracle pins)
DY_Y = [6.0, 1.0625, -10.9375]
DY_HT = [12.0, 0.53125]
DY_H = [[4, 2], [0, 2.125], [12, 0.53125]]
DY_G = {
    "gx": [1.9375, -1.75, 1.5],
    "gdelta": [3.625 * LN2 + 3.875, 4 * LN2 + 0.875, 6.0],
    "gb": [[0.125, 1.875], [7.5, 2.0], [2.0, 0.0]],
    "gc": [[4.0, 2.0], [0.0, -4.25], [6.0, 0.265625]],
    "gA": [-7.375, -2.125],
    "gh0": [0.03125, 0.234375],
}


@pytest.mark.parametrize("lanes", [1, 2])
def test_dyadic_worked_example(gpu, lanes):
    announce(f"dyadic worked example 1x3x1x2, {lanes} lanes per channel")
    t = {k: torch.tensor(v, dtype=torch.float32, device=gpu) for k, v in DYADIC.items()}
    y, hT, H = sscan_fwd(t["x"], t["delta"], t["A"], t["b"], t["c"], t["h0"], return_H=True,
                         plan=Plan(lanes, 1))
    assert_close("y", y, np.array(DY_Y).reshape(1, 3, 1), 1e-6)
    assert_close("hT", hT, np.array(DY_HT).reshape(1, 1, 2), 1e-6)
    assert_close("H", H, np.array(DY_H, dtype=float).reshape(1, 3, 1, 2), 1e-6)
    g = sscan_bwd(t["dy"], t["x"], t["delta"], t["A"], t["b"], t["c"], t["h0"], H, t["dhT"], plan=Plan(lanes, 1))
    for name, got in zip(GRADS, g):
        ref = np.array(DY_G[name], dtype=float).reshape(tuple(got.shape))
        assert_close(name, got, ref, 1e-6)


@pytest.mark.parametrize("layout,with_H", [("lanes", True), ("lanes", False), ("state_groups", False)])
def test_memoryless_limit(gpu, layout, with_H):
    B, T, D, DS = 2, 70, 40, 16
    announce(f"memoryless limit A=-1e6: B={B} T={T} D={D} DS={DS} layout={layout} H={with_H}")
    w = workloads.custom(B, T, D, DS, seed=41, h0_std=0.3, delta_mu=-1.0, with_dy=True, with_dhT=True)
    inp = workloads.make_inputs(w)
    inp["A"] = torch.full_like(inp["A"], -1e6)
    g = to_dev(inp, gpu)
    out = sscan_fwd(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], return_H=with_H, plan=Plan(0, 1, layout))
    y, hT = out[0], out[1]
    e = {k: f64(inp[k]) for k in ("x", "delta", "b", "c")}
    y_closed = e["delta"] * e["x"] * np.einsum("btn,btn->bt", e["b"], e["c"])[:, :, None]
    hT_closed = e["delta"][:, -1, :, None] * e["b"][:, -1, None, :] * e["x"][:, -1, :, None]
    assert_close("y vs delta x <b, c>", y, y_closed, TOL_F32)
    assert_close("hT vs delta b x", hT, hT_closed, TOL_F32)
    yr, hTr = oracle.fwd(inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"])
    assert_close("y", y, yr, TOL_F32)
    assert_close("hT", hT, hTr, TOL_F32)
    if with_H:
        H = out[2]
        # no memory: every state is that step's injection alone
        H_closed = e["delta"][..., None] * e["b"][:, :, None, :] * e["x"][..., None]
        assert_close("H", H, H_closed, TOL_F32)
        grads = sscan_bwd(g["dy"], g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], H, g["dhT"])
        ref = oracle.bwd(inp["dy"], inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"], inp["dhT"])
        for name, a, r in zip(GRADS, grads, ref):
            assert_close(name, a, r, TOL_F32)
        # every decay is 0, so no gradient reaches A or h0
        assert torch.count_nonzero(grads[4]).item() == 0 and torch.count_nonzero(grads[5]).item() == 0


def test_softplus_far_below_zero_single_step(gpu):
    """T = 1 from h0 = 0 with no skip term: y = softplus(r) x <b, c>, so y / (x <b, c>) is
    the kernel's softplus itself; at r = -40 it must equal e^-40 (log(1 + e^r) and e^r
    differ by e^-80 / 2 relative)."""
    B, D, DS = 2, 64, 16
    announce(f"softplus at delta_raw=-40, T=1: B={B} D={D} DS={DS}")
    w = workloads.custom(B, 1, D, DS, seed=42)
    inp = workloads.make_inputs(w)
    inp["c"] = inp["b"].clone()  # <b, b> > 0: no cancellation in the sum over states
    raw = torch.full_like(inp["delta_raw"], -40.0)
    g = to_dev(inp, gpu)
    y, hT = sscan_mamba_fwd(g["x"], raw.to(gpu), g["A_log"], g["b"], g["c"], None, None)
    bc = np.einsum("btn,btn->bt", f64(inp["b"]), f64(inp["c"]))[:, :, None]
    ratio = f64(y) / (f64(inp["x"]) * bc)
    assert np.max(np.abs(ratio / math.exp(-40.0) - 1.0)) < 1e-5


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_softplus_far_below_zero_through_the_wrapper(gpu, io):
    B, T, D, DS = 2, 90, 48, 16
    announce(f"wrapper with delta_raw in [-40, -30]: B={B} T={T} D={D} DS={DS} io={io}")
    w = workloads.custom(B, T, D, DS, io=io, seed=43, h0_std=0.3, delta_mu=-1.0, with_dy=True, with_dhT=True)
    inp = workloads.make_inputs(w)
    gen = torch.Generator().manual_seed(430)
    raw = (-40.0 + 10.0 * torch.rand(inp["delta_raw"].shape, generator=gen)).to(inp["delta_raw"].dtype)
    inp["delta_raw"] = raw
    g = to_dev(inp, gpu)
    # h0 = 0 and no skip term: y is proportional to the tiny steps, so its relative error is the softplus's
    y0, _ = sscan_mamba_fwd(g["x"], g["delta_raw"], g["A_log"], g["b"], g["c"], None, None)
    y0r, _ = oracle.mamba_fwd(inp["x"], inp["delta_raw"], inp["A_log"], inp["b"], inp["c"], None, None)
    assert_close("y (h0 = 0, no skip)", y0, y0r, TOL_F32 if io == "f32" else 2e-2)
    # with h0, the skip term and dhT: all seven gradients (fp32 outputs, 1e-4)
    y, hT, H = sscan_mamba_fwd(g["x"], g["delta_raw"], g["A_log"], g["b"], g["c"], g["Dskip"], g["h0"], return_H=True)
    grads = sscan_mamba_bwd(g["dy"], g["x"], g["delta_raw"], g["A_log"], g["b"], g["c"], g["Dskip"], g["h0"], H,
                            g["dhT"])
    ref = oracle.mamba_bwd(inp["dy"], inp["x"], inp["delta_raw"], inp["A_log"], inp["b"], inp["c"], inp["Dskip"],
                           inp["h0"], inp["dhT"])
    gx, gdr, gAl, gb, gc, gD, gh0 = ref
    for name, a, r in zip(["gx", "gdelta_raw", "gb", "gc", "gA_log", "gh0", "gDskip"], grads,
                          (gx, gdr, gb, gc, gAl, gh0, gD)):
        assert_close(name, a, r, TOL_F32)


def test_inputs_broadcast_over_the_batch(gpu):
    """b, c (and x) given as one batch row expanded over B (batch stride 0 in torch): the
    binding passes a full-stride copy, and the result equals the oracle on the
    materialised inputs."""
    B, T, D, DS = 3, 70, 40, 16
    announce(f"batch-broadcast x, b, c: B={B} T={T} D={D} DS={DS}")
    w = workloads.custom(B, T, D, DS, seed=44, h0_std=0.3, delta_mu=-1.0, with_dy=True, with_dhT=True)
    inp = workloads.make_inputs(w)
    g = to_dev(inp, gpu)
    dense = dict(inp)
    for k in ("x", "b", "c"):
        shape = inp[k].shape
        dense[k] = inp[k][:1].expand(shape).contiguous()   # what the oracle reads
        g[k] = g[k][:1].expand(shape)                       # a stride-0 view on the device
    assert g["b"].stride(0) == 0 and g["x"].stride(0) == 0
    y, hT, H = sscan_fwd(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], return_H=True)
    yr, hTr = oracle.fwd(dense["x"], dense["delta"], dense["A"], dense["b"], dense["c"], dense["h0"])
    assert_close("y", y, yr, TOL_F32)
    assert_close("hT", hT, hTr, TOL_F32)
    grads = sscan_bwd(g["dy"], g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], H, g["dhT"])
    ref = oracle.bwd(dense["dy"], dense["x"], dense["delta"], dense["A"], dense["b"], dense["c"], dense["h0"],
                     dense["dhT"])
    for name, a, r in zip(GRADS, grads, ref):
        assert_close(name, a, r, TOL_F32)


@pytest.mark.parametrize("T,layout", [(2 ** 24 - 64, "state_groups"), (2 ** 24 + 64, "lanes")])
def test_longest_sequences_on_both_sides_of_the_state_group_limit(gpu, T, layout):
    """The state-group forward addresses a batch row's packed b/c with 32-bit offsets and
    runs for T < 2^24; at 2^24 - 64 steps the library's plan is that layout (16 T-chunks of
    about a million steps), at 2^24 + 64 the lanes layout.  Every element of y and hT of
    both against the oracle, over the whole sequence."""
    announce(f"longest sequence 1x{T}x4x4 fp32, {layout} layout")
    assert sscan.sscan_plan_select(1, T, 4, 4).layout == layout
    w = workloads.custom(1, T, 4, 4, io="f32", seed=23, h0_std=0.3, delta_mu=-1.0)
    inp = workloads.make_inputs(w)
    g = to_dev(inp, gpu)
    y, hT = sscan_fwd(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"])
    torch.cuda.synchronize()
    y, hT = y.cpu(), hT.cpu()
    del g
    yr, hTr = oracle.fwd(inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"])
    assert_close("y", y, yr, TOL_F32)
    assert_close("hT", hT, hTr, TOL_F32)


@pytest.mark.parametrize("B,T,D,DS", [(65535, 3, 4, 4), (1, 40, 2 ** 18, 16)])
def test_largest_batch_and_channel_counts(gpu, B, T, D, DS):
    """The largest batch (B = 65535) and channel count (D*DS = 2^22) the library accepts,
    forward writing H and backward with the library's own plans (and at DS = 16 the H-free
    forward and backward): every element of every output against the oracle."""
    announce(f"largest sizes {B}x{T}x{D}x{DS} fp32: forward writing H + backward")
    w = workloads.custom(B, T, D, DS, io="f32", seed=29, h0_std=0.3, delta_mu=-1.0, with_dy=True, with_dhT=True)
    inp = workloads.make_inputs(w)
    g = to_dev(inp, gpu)
    y, hT, H = sscan_fwd(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], return_H=True)
    grads = sscan_bwd(g["dy"], g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], H, g["dhT"])
    torch.cuda.synchronize()
    yr, hTr, Hr = oracle.fwd(inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"], return_H=True)
    assert_close("y", y, yr, TOL_F32)
    assert_close("hT", hT, hTr, TOL_F32)
    assert_close("H", H, Hr, TOL_F32)
    del Hr, H
    ref = oracle.bwd(inp["dy"], inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"], inp["dhT"])
    for name, got, r in zip(GRADS, grads, ref):
        assert_close(name, got, r, TOL_F32)
    if DS >= 8:  # the H-free path (its backward runs 8 or 16 lanes per channel)
        del grads
        y2, hT2, hck = sscan.sscan_fwd_ckpt(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"])
        grads2 = sscan.sscan_bwd_ckpt(g["dy"], g["x"], g["delta"], g["A"], g["b"], g["c"], hck, g["dhT"])
        torch.cuda.synchronize()
        assert_close("y (H-free path)", y2, yr, TOL_F32)
        assert_close("hT (H-free path)", hT2, hTr, TOL_F32)
        for name, got, r in zip(GRADS, grads2, ref):
            assert_close(name + " (H-free path)", got, r, TOL_F32)
