"""GPU parity: libsscan (through its C ABI and the Python binding) against the fp64
oracle on the same seeded inputs.  Tolerance (max|err|/max|ref| per tensor):
1e-4 for fp32 I/O, 2e-2 for bf16 I/O with fp32 state."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import TOL_BF16, TOL_F32, announce, assert_close, f64, rel_err, to_dev, tol_for
from test_oracle_pins import gradient_identity_residuals

pytestmark = pytest.mark.gpu

sscan = pytest.importorskip("selective_state_space_sscan_amd")
from selective_state_space_sscan_amd import Plan, SelectiveScan, sscan_bwd, sscan_fwd  # noqa: E402


def run_fwd(g, plan=None, return_H=False):
    return sscan_fwd(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], return_H=return_H, plan=plan)


# ----------------------------------------------------------------------------- small cases

def test_tiny_workload_matches_golden(gpu):
    announce("tiny_fwd 1x64x16x4 fp32")
    w = workloads.get("tiny_fwd")
    inp = workloads.make_inputs(w)
    y, hT = run_fwd(to_dev(inp, gpu))
    with open(os.path.join(os.path.dirname(__file__), "golden", "tiny_fwd_oracle.json")) as f:
        doc = json.load(f)
    e_y = assert_close("y", y, np.array(doc["y"]).reshape(w.B, w.T, w.D), TOL_F32)
    e_h = assert_close("hT", hT, np.array(doc["hT"]).reshape(w.B, w.D, w.DS), TOL_F32)
    print(f"tiny_fwd: y rel err {e_y:.2e}, hT rel err {e_h:.2e}")


def test_selftest_shape_forward_backward(gpu):
    announce("selftest 2x7x64x16 fp32 fwd+bwd with dhT")
    w = workloads.get("selftest", with_dhT=True)
    inp = workloads.make_inputs(w)
    g = to_dev(inp, gpu)
    y, hT, H = run_fwd(g, return_H=True)
    yr, hTr, Hr = oracle.fwd(inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"], return_H=True)
    assert_close("y", y, yr, TOL_F32)
    assert_close("hT", hT, hTr, TOL_F32)
    assert_close("H", H, Hr, TOL_F32)
    grads = sscan_bwd(g["dy"], g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], H, g["dhT"])
    ref = oracle.bwd(inp["dy"], inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"], inp["dhT"])
    for name, a, r in zip(["gx", "gdelta", "gb", "gc", "gA", "gh0"], grads, ref):
        assert_close(name, a, r, TOL_F32)


SMALL_FWD = [
    # B, T, D, DS, io, h0, lanes, chunks
    (1, 1, 1, 1, "f32", True, 0, 0),
    (2, 5, 3, 2, "f32", True, 0, 0),
    (2, 77, 19, 4, "f32", True, 0, 0),
    (3, 130, 70, 8, "bf16", True, 0, 0),
    (2, 200, 33, 16, "f32", False, 0, 0),
    (1, 300, 300, 16, "bf16", True, 0, 0),
    (2, 129, 65, 16, "f32", True, 1, 1),
    (2, 129, 65, 16, "f32", True, 2, 1),
    (2, 129, 65, 16, "f32", True, 4, 1),
    (2, 129, 65, 16, "bf16", True, 8, 1),
    (2, 129, 65, 16, "f32", True, 16, 1),
    (2, 257, 40, 16, "f32", True, 16, 3),
    (2, 257, 40, 8, "bf16", True, 4, 5),
    (1, 1000, 17, 16, "f32", True, 8, 7),
    (2, 64, 300, 4, "f32", False, 2, 2),
    (1, 9, 5, 1, "f32", True, 1, 4),
]


@pytest.mark.parametrize("B,T,D,DS,io,h0,lanes,chunks", SMALL_FWD)
def test_forward_small_shapes(gpu, B, T, D, DS, io, h0, lanes, chunks):
    announce(f"fwd B={B} T={T} D={D} DS={DS} io={io} h0={h0} plan=({lanes},{chunks})")
    w = workloads.custom(B, T, D, DS, io=io, seed=B * 1000 + T + D + DS, h0_std=0.3 if h0 else 0.0, delta_mu=-1.0)
    inp = workloads.make_inputs(w)
    y, hT, H = run_fwd(to_dev(inp, gpu), plan=Plan(lanes, chunks), return_H=True)
    yr, hTr, Hr = oracle.fwd(inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"], return_H=True)
    assert y.dtype == inp["x"].dtype
    assert_close("y", y, yr, tol_for(io))
    assert_close("hT", hT, hTr, TOL_F32)
    assert_close("H", H, Hr, TOL_F32)


SMALL_BWD = [
    (1, 1, 1, 1, "f32", True, True, 0),
    (2, 6, 3, 4, "f32", True, True, 0),
    (2, 45, 21, 16, "f32", True, True, 0),
    (2, 70, 37, 8, "f32", False, False, 0),
    (3, 33, 100, 16, "f32", True, False, 4),
    (2, 64, 64, 16, "f32", True, True, 1),
    (2, 64, 64, 16, "f32", True, True, 2),
    (2, 64, 64, 16, "f32", True, True, 8),
    (1, 100, 300, 2, "f32", True, True, 0),
    (2, 50, 40, 16, "bf16", True, True, 0),
]


@pytest.mark.parametrize("B,T,D,DS,io,h0,dhT,lanes", SMALL_BWD)
def test_backward_small_shapes(gpu, B, T, D, DS, io, h0, dhT, lanes):
    announce(f"bwd B={B} T={T} D={D} DS={DS} io={io} h0={h0} dhT={dhT} lanes={lanes}")
    w = workloads.custom(B, T, D, DS, io=io, seed=7 + B * 100 + T + D, h0_std=0.3 if h0 else 0.0, delta_mu=-1.0,
                         with_dy=True, with_dhT=dhT)
    inp = workloads.make_inputs(w)
    g = to_dev(inp, gpu)
    y, hT, H = run_fwd(g, return_H=True)
    grads = sscan_bwd(g["dy"], g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], H, g["dhT"], plan=Plan(lanes, 0))
    # bf16 I/O: the backward consumes the GPU's own fp32 H, so compare with fp32 tolerance except
    # where the bf16 inputs themselves enter (they are the same bf16 values on both sides).
    ref = oracle.bwd(inp["dy"], inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"], inp["dhT"])
    for name, a, r in zip(["gx", "gdelta", "gb", "gc", "gA", "gh0"], grads, ref):
        assert_close(name, a, r, TOL_F32)


CHUNKED_BWD = [
    # B, T, D, DS, io, h0, dhT, lanes, chunks
    (2, 300, 40, 16, "f32", True, True, 16, 2),
    (2, 300, 40, 16, "f32", True, False, 16, 3),
    (1, 1000, 33, 16, "f32", False, True, 16, 5),
    (2, 257, 70, 8, "f32", True, True, 8, 2),
    (2, 513, 20, 4, "bf16", True, True, 4, 4),
    (1, 128, 16, 16, "f32", True, True, 16, 4),
    # four lanes per channel (the default), ragged T and D, two and eight sub-chunks per chunk
    (2, 1000, 100, 16, "f32", True, True, 4, 8),
    (1, 2048, 70, 16, "bf16", True, True, 4, 4),
]


@pytest.mark.parametrize("B,T,D,DS,io,h0,dhT,lanes,chunks", CHUNKED_BWD)
def test_backward_chunked_sweep(gpu, B, T, D, DS, io, h0, dhT, lanes, chunks):
    announce(f"chunked bwd B={B} T={T} D={D} DS={DS} io={io} h0={h0} dhT={dhT} plan=({lanes},{chunks})")
    w = workloads.custom(B, T, D, DS, io=io, seed=11 + T + D, h0_std=0.3 if h0 else 0.0, delta_mu=-1.0,
                         with_dy=True, with_dhT=dhT)
    inp = workloads.make_inputs(w)
    g = to_dev(inp, gpu)
    y, hT, H = run_fwd(g, return_H=True)
    grads = sscan_bwd(g["dy"], g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], H, g["dhT"],
                      plan=Plan(lanes, chunks))
    ref = oracle.bwd(inp["dy"], inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"], inp["dhT"])
    for name, a, r in zip(["gx", "gdelta", "gb", "gc", "gA", "gh0"], grads, ref):
        assert_close(name, a, r, TOL_F32)
    single = sscan_bwd(g["dy"], g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], H, g["dhT"],
                       plan=Plan(lanes, 1))
    for name, a, r in zip(["gx", "gdelta", "gb", "gc", "gA", "gh0"], grads, single):
        assert rel_err(a, r) < 1e-5, name


def test_zero_delta_keeps_state_bitwise(gpu):
    announce("delta=0: hT == h0 bitwise")
    w = workloads.custom(2, 50, 40, 16, seed=3, h0_std=0.5)
    inp = workloads.make_inputs(w)
    inp["delta"] = torch.zeros_like(inp["delta"])
    g = to_dev(inp, gpu)
    for plan in (Plan(16, 1), Plan(4, 1), Plan(16, 3)):
        y, hT = run_fwd(g, plan=plan)
        assert torch.equal(hT.cpu(), inp["h0"]), plan
        y_ref = np.einsum("bdn,btn->btd", f64(inp["h0"]), f64(inp["c"]))
        assert_close("y", y, y_ref, TOL_F32)


def test_empty_and_degenerate_sizes(gpu):
    announce("T=0, B=0, D=0")
    w = workloads.custom(2, 0, 8, 4, seed=4, h0_std=0.5, with_dy=True, with_dhT=True)
    inp = workloads.make_inputs(w)
    g = to_dev(inp, gpu)
    y, hT = run_fwd(g)
    assert y.shape == (2, 0, 8) and torch.equal(hT.cpu(), inp["h0"])
    g0 = {k: v for k, v in g.items()}
    g0["h0"] = None
    y, hT = run_fwd(g0)
    assert torch.count_nonzero(hT).item() == 0
    H = torch.empty((2, 0, 8, 4), device=gpu)
    gx, gd, gb, gc, gA, gh0 = sscan_bwd(g["dy"], g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], H, g["dhT"])
    assert torch.count_nonzero(gA).item() == 0 and torch.equal(gh0.cpu(), inp["dhT"])
    wb = workloads.custom(0, 5, 8, 4, seed=5)
    gb0 = to_dev(workloads.make_inputs(wb), gpu)
    y, hT = run_fwd(gb0)
    assert y.shape == (0, 5, 8) and hT.shape == (0, 8, 4)


def test_split_calls_carry_the_state(gpu):
    announce("three calls with h0 <- hT vs one oracle pass; batch-strided T-slices")
    w = workloads.custom(2, 300, 70, 16, io="bf16", seed=6, h0_std=0.1)
    inp = workloads.make_inputs(w)
    g = to_dev(inp, gpu)
    y_all = torch.empty_like(g["x"])
    h = g["h0"]
    for t0, t1 in [(0, 100), (100, 101), (101, 300)]:
        sl = slice(t0, t1)
        _, h = sscan_fwd(g["x"][:, sl], g["delta"][:, sl], g["A"], g["b"][:, sl], g["c"][:, sl], h, y=y_all[:, sl])
    yr, hTr = oracle.fwd(inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"])
    assert_close("y", y_all, yr, TOL_BF16)
    assert_close("hT", h, hTr, TOL_F32)
    # and against the GPU's own single call: identical up to fp32 rounding of the state
    y1, h1 = run_fwd(g, plan=Plan(0, 1))
    assert rel_err(h, h1) < 1e-6


def test_split_calls_backward_chains_dhT(gpu):
    """A sequence split over three forward calls is back-propagated call by call, last
    call first, each call's gh0 becoming the previous call's dhT; the result equals the
    backward of one unsplit call."""
    announce("split-call backward: gh0 -> dhT across 3 calls, 2x300x40x16 fp32")
    w = workloads.custom(2, 300, 40, 16, seed=13, h0_std=0.2, with_dy=True, with_dhT=True)
    inp = workloads.make_inputs(w)
    g = to_dev(inp, gpu)
    bounds = [(0, 90), (90, 91), (91, 300)]
    hs, Hs = [g["h0"]], []
    for t0, t1 in bounds:
        sl = slice(t0, t1)
        _, hT, H = sscan_fwd(g["x"][:, sl], g["delta"][:, sl], g["A"], g["b"][:, sl], g["c"][:, sl], hs[-1],
                             return_H=True)
        hs.append(hT)
        Hs.append(H)
    dhT = g["dhT"]
    gx = torch.empty_like(g["x"])
    gd = torch.empty_like(g["x"])
    gb = torch.empty_like(g["b"])
    gc = torch.empty_like(g["c"])
    gA = torch.zeros_like(g["A"])
    for k in reversed(range(len(bounds))):
        t0, t1 = bounds[k]
        sl = slice(t0, t1)
        r = sscan_bwd(g["dy"][:, sl], g["x"][:, sl], g["delta"][:, sl], g["A"], g["b"][:, sl], g["c"][:, sl],
                      hs[k], Hs[k], dhT)
        gx[:, sl], gd[:, sl], gb[:, sl], gc[:, sl] = r[0], r[1], r[2], r[3]
        gA += r[4]
        dhT = r[5]
    ref = oracle.bwd(inp["dy"], inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"], inp["dhT"])
    for name, a, r in zip(["gx", "gdelta", "gb", "gc", "gA", "gh0"], [gx, gd, gb, gc, gA, dhT], ref):
        assert_close(name, a, r, TOL_F32)


def test_backward_is_bitwise_reproducible(gpu):
    announce("bwd determinism 2x256x96x16")
    w = workloads.custom(2, 256, 96, 16, seed=8, h0_std=0.1, with_dy=True, with_dhT=True)
    g = to_dev(workloads.make_inputs(w), gpu)
    y, hT, H = run_fwd(g, return_H=True)
    a = sscan_bwd(g["dy"], g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], H, g["dhT"])
    b = sscan_bwd(g["dy"], g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], H, g["dhT"])
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    y2, hT2, H2 = run_fwd(g, return_H=True)
    assert torch.equal(y, y2) and torch.equal(hT, hT2) and torch.equal(H, H2)


@pytest.mark.parametrize("io,chunks", [("f32", 3), ("bf16", 1)])
def test_four_lane_sweep_reads_every_fourth_row_of_H(gpu, io, chunks):
    """With four states per lane the sweep reads H only at rows r = 3 (mod 4) (the state
    entering each four-step block) and at the last step, and re-forms the rows between
    with the forward's own update: poisoning every other row with NaN must leave the
    gradients bitwise unchanged (and they match the oracle in the parity tests)."""
    B, T, D, DS = 2, 203, 70, 16
    announce(f"four-lane sweep, poisoned H rows: B={B} T={T} D={D} DS={DS} io={io} chunks={chunks}")
    w = workloads.custom(B, T, D, DS, io=io, seed=77, h0_std=0.3, delta_mu=-1.0, with_dy=True, with_dhT=True)
    inp = workloads.make_inputs(w)
    g = to_dev(inp, gpu)
    y, hT, H = run_fwd(g, return_H=True)
    plan = Plan(4, chunks)
    ref = sscan_bwd(g["dy"], g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], H, g["dhT"], plan=plan)
    Hp = H.clone()
    rows = torch.arange(T, device=gpu)
    unread = (rows % 4 != 3) & (rows != T - 1)
    Hp[:, unread] = float("nan")
    got = sscan_bwd(g["dy"], g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], Hp, g["dhT"], plan=plan)
    torch.cuda.synchronize()
    for name, a, b in zip(["gx", "gdelta", "gb", "gc", "gA", "gh0"], got, ref):
        assert torch.equal(a, b), name


def test_autograd_function(gpu):
    announce("SelectiveScan autograd 2x40x24x8")
    w = workloads.custom(2, 40, 24, 8, seed=9, h0_std=0.2, with_dy=True, with_dhT=True)
    inp = workloads.make_inputs(w)
    g = to_dev(inp, gpu)
    leaves = {k: g[k].clone().requires_grad_(True) for k in ("x", "delta", "A", "b", "c", "h0")}
    y, hT = SelectiveScan.apply(leaves["x"], leaves["delta"], leaves["A"], leaves["b"], leaves["c"], leaves["h0"])
    L = (y * g["dy"]).sum() + (hT * g["dhT"]).sum()
    L.backward()
    ref = oracle.bwd(inp["dy"], inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"], inp["dhT"])
    for name, key, r in zip(["gx", "gdelta", "gb", "gc", "gA", "gh0"], ["x", "delta", "b", "c", "A", "h0"], ref):
        assert_close(name, leaves[key].grad, r, TOL_F32)


# ----------------------------------------------------------------------------- full sizes

def test_fwd_f32_full(gpu):
    w = workloads.get("fwd_f32")
    announce(f"{w.name}: {w.note} (automatic plan)")
    inp = workloads.make_inputs(w)
    y, hT = run_fwd(to_dev(inp, gpu))
    yr, hTr = oracle.fwd(inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"])
    e_y = assert_close("y", y, yr, TOL_F32)
    e_h = assert_close("hT", hT, hTr, TOL_F32)
    print(f"fwd_f32 full: y rel err {e_y:.2e}, hT rel err {e_h:.2e}")


def test_fwd_bf16_full(gpu):
    w = workloads.get("fwd_bf16")
    announce(f"{w.name}: {w.note} (automatic plan, full oracle)")
    inp = workloads.make_inputs(w)
    y, hT = run_fwd(to_dev(inp, gpu))
    yr, hTr = oracle.fwd(inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"])
    e_y = assert_close("y", y, yr, TOL_BF16)
    e_h = assert_close("hT", hT, hTr, TOL_F32)
    print(f"fwd_bf16 full: y rel err {e_y:.2e}, hT rel err {e_h:.2e}")


def test_long_chunked_bf16_full(gpu):
    """4x16384x2048x16 bf16 run as 8 calls of 2048 steps with hT -> h0: every element of y
    and hT against ONE unchunked oracle pass over the whole sequence (pssa_kernels.py page,
    module docstring: h0 and hT carry the state across chunks), and against the GPU's own
    single call over all 16384 steps.  The calls hand over the fp32 state exactly, and both
    run the same kernel with the same per-step operations, so the two GPU results must be
    bitwise equal."""
    w = workloads.get("long_chunked_bf16")
    announce(f"{w.name}: {w.note}; every element vs one unchunked oracle pass and vs one GPU call")
    inp = workloads.make_inputs(w)
    g = to_dev(inp, gpu)
    y_all = torch.empty_like(g["x"])
    h = g["h0"]
    for t0, t1 in workloads.chunk_bounds(w.T, w.chunks):
        sl = slice(t0, t1)
        _, h = sscan_fwd(g["x"][:, sl], g["delta"][:, sl], g["A"], g["b"][:, sl], g["c"][:, sl], h, y=y_all[:, sl])
    y1, h1 = run_fwd(g)  # one call over all T = 16384 steps
    torch.cuda.synchronize()
    assert torch.equal(y_all, y1), "8 calls and one call differ in y"
    assert torch.equal(h, h1), "8 calls and one call differ in hT"
    del y1, h1, g
    yr, hTr = oracle.fwd(inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"])
    e_y = assert_close("y (all 4x16384x2048)", y_all, yr, TOL_BF16)
    del yr
    e_h = assert_close("hT", h, hTr, TOL_F32)
    print(f"long_chunked_bf16 full: y rel err {e_y:.2e}, hT rel err {e_h:.2e}")


def test_fwd_bwd_f32_full(gpu):
    w = workloads.get("fwd_bwd_f32")
    announce(f"{w.name}: {w.note} (automatic plans, full oracle)")
    inp = workloads.make_inputs(w)
    g = to_dev(inp, gpu)
    y, hT, H = run_fwd(g, return_H=True)
    grads = sscan_bwd(g["dy"], g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], H, None)
    torch.cuda.synchronize()
    yr, hTr, Hr = oracle.fwd(inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"], return_H=True)
    e_y = assert_close("y", y, yr, TOL_F32)
    e_h = assert_close("hT", hT, hTr, TOL_F32)
    e_H = assert_close("H", H, Hr, TOL_F32)  # every state of every step
    print(f"fwd_bwd full: y rel err {e_y:.2e}, hT rel err {e_h:.2e}, H rel err {e_H:.2e}")
    del Hr
    ref = oracle.bwd(inp["dy"], inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"], None)
    errs = {}
    for name, a, r in zip(["gx", "gdelta", "gb", "gc", "gA", "gh0"], grads, ref):
        errs[name] = assert_close(name, a, r, TOL_F32)
    print("fwd_bwd full rel errs: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    # gc from the GPU's own H in fp64: the backward's channel sums agree with its forward states
    Hd = f64(H)
    gc_from_H = np.einsum("btd,btdn->btn", f64(inp["dy"]), Hd)
    assert_close("gc vs sum_d dy*H", grads[3], gc_from_H, 1e-5)
    del Hd, gc_from_H
    # the four exact relations between the gradients that invariances of the map give (they
    # hold at any size), evaluated on the GPU's own outputs
    e = {k: f64(inp[k]) for k in ("x", "delta", "A", "b", "c", "h0", "dy")}
    e["dhT"] = None
    res = gradient_identity_residuals(e, f64(y), f64(hT), [f64(t) for t in grads])
    print("fwd_bwd full gradient identity residuals: " + " ".join(f"{r:.1e}" for r in res))
    assert max(res) < 1e-5, res


# Shapes where the library's own plans take the branches of its plan rules: the forward in
# the state-group layout split into T-chunks (one pass would have under 512 compute waves),
# the forward keeping boundary states likewise, and the backward's four states per lane
# below DS = 16.  Whole-tensor parity of every output against the oracle.
AUTO_PLAN_CASES = [
    # B, T, D, DS, io, (fwd layout, fwd chunks), bwd lanes
    (1, 4096, 256, 16, "f32", ("state_groups", 16), 4),
    (2, 4096, 128, 8, "bf16", ("state_groups", 16), 8),
    (8, 256, 2048, 4, "f32", ("state_groups", 1), 1),
    (8, 256, 1024, 8, "f32", ("state_groups", 1), 2),
]


@pytest.mark.parametrize("B,T,D,DS,io,fplan,blanes", AUTO_PLAN_CASES)
def test_library_plans_at_their_rule_branches(gpu, B, T, D, DS, io, fplan, blanes):
    from selective_state_space_sscan_amd import sscan_bwd_ckpt, sscan_fwd_ckpt, sscan_plan_select
    w = workloads.custom(B, T, D, DS, io=io, seed=400 + DS, h0_std=0.2, delta_mu=-1.0, with_dy=True, with_dhT=True)
    inp = workloads.make_inputs(w)
    g = to_dev(inp, gpu)
    dt = g["x"].dtype
    pf, pk, pb = (sscan_plan_select(B, T, D, DS, dt), sscan_plan_select(B, T, D, DS, dt, ckpt=True),
                  sscan_plan_select(B, T, D, DS, dt, backward=True))
    announce(f"library plans B={B} T={T} D={D} DS={DS} {io}: fwd {pf} ckpt {pk} bwd {pb}")
    assert (pf.layout, pf.chunks) == fplan and (pk.layout, pk.chunks) == fplan and pb.lanes == blanes
    y, hT = sscan_fwd(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"])
    yk, hTk, hck = sscan_fwd_ckpt(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"])
    _, _, H = sscan_fwd(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], return_H=True)
    grads = sscan_bwd(g["dy"], g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], H, g["dhT"])
    gk = sscan_bwd_ckpt(g["dy"], g["x"], g["delta"], g["A"], g["b"], g["c"], hck, g["dhT"]) if DS >= 8 else None
    torch.cuda.synchronize()
    yr, hTr = oracle.fwd(inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"])
    assert_close("y", y, yr, tol_for(io))
    assert_close("hT", hT, hTr, TOL_F32)
    assert_close("y (boundary states kept)", yk, yr, tol_for(io))
    assert torch.equal(hTk, hT)  # the same layout and chunks: the same states
    ref = oracle.bwd(inp["dy"], inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"], inp["dhT"])
    for name, a, r in zip(["gx", "gdelta", "gb", "gc", "gA", "gh0"], grads, ref):
        assert_close(name, a, r, TOL_F32)
    if gk is not None:
        for name, a, r in zip(["gx", "gdelta", "gb", "gc", "gA", "gh0"], gk, ref):
            assert_close(name + " (H-free)", a, r, TOL_F32)
