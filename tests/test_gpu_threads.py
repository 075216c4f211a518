"""Concurrent calls (the header's contract: calls are thread-safe when they use distinct
workspaces and outputs): four host threads, each on a stream of its own, run the forward
writing H and the backward on their own inputs at the same time; every result must equal,
bit for bit, the same calls made one after another on one stream."""
import threading

import pytest
import torch

import workloads
from parity import announce, to_dev

pytestmark = pytest.mark.gpu

sscan = pytest.importorskip("selective_state_space_sscan_amd")
from selective_state_space_sscan_amd import sscan_bwd, sscan_fwd  # noqa: E402


def run_pair(g):
    y, hT, H = sscan_fwd(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], return_H=True)
    grads = sscan_bwd(g["dy"], g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], H, g["dhT"])
    return (y, hT, H) + tuple(grads)


def test_concurrent_calls_from_threads_on_their_own_streams(gpu):
    shapes = [(2, 300, 256, 16, "f32"), (4, 200, 512, 16, "bf16"), (1, 700, 96, 8, "f32"), (3, 129, 64, 4, "f32")]
    announce(f"four threads on four streams: {shapes}")
    inputs = []
    for k, (B, T, D, DS, io) in enumerate(shapes):
        w = workloads.custom(B, T, D, DS, io=io, seed=300 + k, h0_std=0.3, delta_mu=-1.0, with_dy=True,
                             with_dhT=True)
        inputs.append(to_dev(workloads.make_inputs(w), gpu))
    serial = [run_pair(g) for g in inputs]
    torch.cuda.synchronize()

    results = [None] * len(inputs)
    failures = []
    start = threading.Barrier(len(inputs))

    def worker(k):
        try:
            s = torch.cuda.Stream(device=gpu)
            start.wait()
            with torch.cuda.stream(s):
                out = None
                for _ in range(3):  # several calls each, so the threads' calls interleave
                    out = run_pair(inputs[k])
            s.synchronize()
            results[k] = out
        except Exception as e:  # reported in the main thread
            failures.append((k, repr(e)))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(len(inputs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not failures, failures
    names = ["y", "hT", "H", "gx", "gdelta", "gb", "gc", "gA", "gh0"]
    for k, (a, b) in enumerate(zip(serial, results)):
        for name, u, v in zip(names, a, b):
            assert torch.equal(u, v), f"thread {k}: {name} differs from the serial call"
