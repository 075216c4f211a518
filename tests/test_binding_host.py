"""Host-side checks of the Python binding's argument marshalling: batch strides of
broadcast (expanded) tensors and caller-supplied fp32 outputs.  No GPU is used: these
helpers only inspect tensor metadata, and every bad argument raises before any call
into the library."""
import pytest
import torch

from selective_state_space_sscan_amd import api


def test_batch_stride_of_contiguous_and_sliced_tensors():
    t = torch.zeros(4, 10, 3)
    assert api._batch_stride(t, "t") == 30
    # a T-slice of a longer sequence keeps the long batch stride (no copy)
    assert api._batch_stride(t[:, 2:5], "t") == 30
    # one batch row: the stride is irrelevant and reported as one row
    assert api._batch_stride(torch.zeros(1, 10, 3), "t") == 30


def test_batch_stride_rejects_rows_broadcast_over_the_batch():
    e = torch.zeros(1, 64, 16).expand(4, 64, 16)
    assert e.stride(0) == 0
    with pytest.raises(ValueError, match="batch rows overlap"):
        api._batch_stride(e, "b")


def test_rows_view_copies_broadcast_rows():
    base = torch.randn(1, 64, 16)
    e = base.expand(4, 64, 16)
    t, s = api._rows_view(e, "b")
    assert s == 64 * 16 and t.is_contiguous()
    assert torch.equal(t, base.expand(4, 64, 16))


def test_same_stride_on_two_expanded_tensors_gives_a_full_batch_stride():
    b = torch.randn(1, 64, 16).expand(4, 64, 16)
    c = torch.randn(1, 64, 16).expand(4, 64, 16)
    (b2, c2), bs = api._same_stride([b, c], ["b", "c"])
    assert bs == 64 * 16
    for t in (b2, c2):
        assert t.stride(0) == 64 * 16 and t.is_contiguous()


def test_same_stride_mixed_slice_and_expand():
    x = torch.randn(3, 20, 8)[:, 5:15]            # batch stride 160, rows of 80
    d = torch.randn(1, 10, 8).expand(3, 10, 8)     # batch stride 0
    (x2, d2), bs = api._same_stride([x, d], ["x", "delta"])
    assert bs == 80 and x2.is_contiguous() and d2.is_contiguous()


def test_batch_stride_rejects_broadcast_inner_dimensions_and_view_copies_them():
    e = torch.randn(2, 1, 16).expand(2, 64, 16)  # stride 0 along T
    with pytest.raises(ValueError, match="contiguous"):
        api._batch_stride(e, "b")
    t, s = api._rows_view(e, "b")
    assert s == 64 * 16 and t.is_contiguous()


@pytest.mark.parametrize("bad,match", [
    (torch.empty(2, 8, 4, dtype=torch.bfloat16), "float32"),
    (torch.empty(2, 8, 5), "shape"),
    (torch.empty(2, 4, 8).transpose(1, 2), "not contiguous"),
    (torch.empty(1, 8, 4).expand(2, 8, 4), "not contiguous"),
])
def test_supplied_fp32_outputs_are_checked(bad, match):
    """hT (and H, hck) given by the caller: a bf16, wrongly shaped or strided tensor
    would take B*D*DS fp32 stores past its storage, so it is refused."""
    with pytest.raises(ValueError, match=match):
        api._f32_out(bad, (2, 8, 4), "hT")


def test_supplied_fp32_output_passes_through():
    t = torch.empty(2, 8, 4)
    assert api._f32_out(t, (2, 8, 4), "hT") is t
    assert api._f32_out(None, (2, 8, 4), "hT") is None


def test_workspace_sizes_are_remembered_per_shape_plan_and_device(monkeypatch):
    """The binding asks the library for a workspace size once per (entry point, device,
    shape, strides, plan) and reuses the answer: every remembered size equals a fresh
    query, and shapes or plans that differ get entries of their own."""
    import ctypes

    from selective_state_space_sscan_amd import _lib
    lib = _lib.load()
    monkeypatch.setattr(api, "_call", lambda device, fn, *args: fn(*args))
    monkeypatch.setattr(api, "_ws_cache", {})
    dev = torch.device("cpu")
    fwd_cases = [(8, 1024, 256, 16, None), (8, 1024, 256, 16, api.Plan(8, 4, "lanes")), (2, 300, 70, 16, None),
                 (1, 4096, 256, 16, api.Plan(0, 16, "state_groups")), (2, 50, 7, 2, None)]
    bwd_cases = [(8, 1024, 256, 16, None), (8, 1024, 256, 16, api.Plan(16, 2)), (2, 300, 70, 16, None),
                 (2, 50, 8, 8, api.Plan(8, 1))]
    for rep in range(2):
        for B, T, D, DS, plan in fwd_cases:
            d = api._desc(B, T, D, DS, 0)
            _, pp = api._plan_ptr(plan)
            got = api._ws_bytes(dev, "fwd", lib.sscan_fwd_workspace, d, plan, pp)
            assert got == api.sscan_fwd_workspace(B, T, D, DS, torch.float32, plan)
        for B, T, D, DS, plan in bwd_cases:
            d = api._desc(B, T, D, DS, 0)
            _, pp = api._plan_ptr(plan)
            got = api._ws_bytes(dev, "bwd", lib.sscan_bwd_workspace, d, plan, pp)
            assert got == api.sscan_bwd_workspace(B, T, D, DS, torch.float32, plan)
            got = api._ws_bytes(dev, "bwd_ckpt", lib.sscan_bwd_ckpt_workspace, d, plan, pp, 1)
            n = ctypes.c_size_t(0)
            _lib.check(lib.sscan_bwd_ckpt_workspace(ctypes.byref(d), pp, 1, ctypes.byref(n)))
            assert got == n.value
        assert len(api._ws_cache) == len(fwd_cases) + 2 * len(bwd_cases)
