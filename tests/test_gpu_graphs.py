"""A training step captured in a HIP graph: the forward writing H (two-level scan in the
lanes layout, and the state-group layout with its packing kernel) and the backward (local
pass, sweep and partial-sum reduce), with caller-supplied outputs and workspaces.  The
library enqueues only kernels (no memsets or copies), so the captured step is replayed
several times, with eager work and synchronisations in between, and every replay must
equal the eager calls bit for bit."""
import pytest
import torch

import workloads
from parity import announce, to_dev

pytestmark = pytest.mark.gpu

sscan = pytest.importorskip("selective_state_space_sscan_amd")
from selective_state_space_sscan_amd import (Plan, sscan_bwd, sscan_bwd_workspace, sscan_fwd,  # noqa: E402
                                             sscan_fwd_workspace)


@pytest.mark.parametrize("B,T,D,DS,fplan,bplan", [
    (8, 1024, 256, 16, Plan(8, 8, "lanes"), Plan(4, 8)),         # both sides split into T-chunks
    (2, 600, 1024, 16, Plan(0, 1, "state_groups"), Plan(0, 0)),  # H through LDS and store waves
])
def test_training_step_replays_in_a_graph(gpu, B, T, D, DS, fplan, bplan):
    announce(f"graph-captured fwd+bwd {B}x{T}x{D}x{DS} fwd {fplan} bwd {bplan}, 3 replays")
    w = workloads.custom(B, T, D, DS, io="f32", seed=77, h0_std=0.3, delta_mu=-1.0, with_dy=True, with_dhT=True)
    g = to_dev(workloads.make_inputs(w), gpu)
    f32 = dict(dtype=torch.float32, device=gpu)
    y, hT, H = torch.empty(B, T, D, **f32), torch.empty(B, D, DS, **f32), torch.empty(B, T, D, DS, **f32)
    grads = (torch.empty(B, T, D, **f32), torch.empty(B, T, D, **f32), torch.empty(B, T, DS, **f32),
             torch.empty(B, T, DS, **f32), torch.empty(D, DS, **f32), torch.empty(B, D, DS, **f32))
    wsf = torch.empty(max(1, sscan_fwd_workspace(B, T, D, DS, torch.float32, fplan)), dtype=torch.uint8, device=gpu)
    wsb = torch.empty(max(1, sscan_bwd_workspace(B, T, D, DS, torch.float32, bplan)), dtype=torch.uint8, device=gpu)

    def step():
        sscan_fwd(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], y=y, hT=hT, H=H, plan=fplan, workspace=wsf)
        sscan_bwd(g["dy"], g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], H, g["dhT"], plan=bplan,
                  workspace=wsb, out=grads)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (y, hT, H) + grads]

    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream(device=gpu)
    cap.wait_stream(torch.cuda.current_stream(gpu))
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            step()
    torch.cuda.current_stream(gpu).wait_stream(cap)
    torch.cuda.synchronize()
    names = ["y", "hT", "H", "gx", "gdelta", "gb", "gc", "gA", "gh0"]
    for r in range(3):
        for t in (y, hT, H) + grads:  # eager work between replays
            t.fill_(float("nan"))
        wsb.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, t, want in zip(names, (y, hT, H) + grads, ref):
            assert torch.equal(t, want), f"replay {r}: {name} differs from the eager step"
