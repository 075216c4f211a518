"""Pins for the fp64 oracle: results fixed by the definition and by mathematics,
not by re-running the oracle's own formula.

Definition ("pssa-100m/pssa_kernels.py" page, module docstring):
    h_t = exp(delta_t * A) * h_{t-1} + delta_t * b_t * x_t,   y_t = <h_t, c_t>,
    h_{-1} = h0, hT = h_{T-1};  A (D,DS) negative, delta (B,T,D) positive, b, c (B,T,DS).
The gradient pins use L = sum(dy * y) + sum(dhT * hT); the page's scan_bwd computes
the dhT = 0 case of that adjoint.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")

LN2 = math.log(2.0)


def rel_err(a, ref):
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(a - ref)) if ref.size else 0.0
    return num / den if den > 0 else num


def rand_case(B, T, D, DS, seed, h0=True, dhT=False, delta_mu=-1.0):
    w = workloads.custom(B, T, D, DS, seed=seed, delta_mu=delta_mu, h0_std=0.3 if h0 else 0.0,
                         with_dy=True, with_dhT=dhT)
    inp = workloads.make_inputs(w)
    return {k: (None if v is None else v.double().numpy()) for k, v in inp.items()}


# ---------------------------------------------------------------------------
# A worked example derived by hand from the definition.  A = [-ln2, -2 ln2] and
# delta in {1, 2} make every decay a power of 1/2, so every value is a dyadic
# rational (gdelta carries an exact multiple of ln 2).
#   decays a_t = [2^-d_t, 4^-d_t]:  t0 [1/2, 1/4], t1 [1/4, 1/16], t2 [1/2, 1/4]
#   u_t = d_t x_t b_t:               t0 [2, 4],    t1 [-1, 2],     t2 [12, 0]
#   h_0 = [2+2, -2+4] = [4, 2];  h_1 = [1-1, 2/16+2] = [0, 2.125];
#   h_2 = [0+12, 2.125/4+0] = [12, 0.53125]
#   y = [4+2, 2.125*0.5, -12+2*0.53125] = [6, 1.0625, -10.9375]
# Backward with dy = [1, -2, 0.5], dhT = [1, -1]:
#   t2: g = 0.5*[-1,2] + [1,-1] = [0.5, 0];  S = 1.5;  gx = 1.5;  gdelta = 0 + 4*1.5 = 6
#       gb = g*d*x = [2, 0];  gc = dy*h_2 = [6, 0.265625];  gA += g*h_1*a*d = [0, 0];  G = a*g = [0.25, 0]
#   t1: g = -2*[2,0.5] + [0.25,0] = [-3.75, -1];  S = -1.875 + 1 = -0.875;  gx = 2*S = -1.75
#       sum_n A a g h_0 = -ln2*(1/4)(-3.75)(4) - 2ln2*(1/16)(-1)(2) = 4 ln2;  gdelta = 4 ln2 + 0.875
#       gb = g*(-2) = [7.5, 2];  gc = -2*h_1 = [0, -4.25];  gA += [(-3.75)(4)(1/4)(2), (-1)(2)(1/16)(2)] = [-7.5, -0.25]
#       G = [-0.9375, -0.0625]
#   t0: g = [1,1] + G = [0.0625, 0.9375];  S = 0.0625 + 1.875 = 1.9375;  gx = 1.9375
#       sum_n A a g h0 = -ln2*(1/2)(0.0625)(4) - 2ln2*(1/4)(0.9375)(-8) = 3.625 ln2;  gdelta = 3.625 ln2 + 3.875
#       gb = 2g = [0.125, 1.875];  gc = h_0 = [4, 2];  gA += [0.125, -1.875];  gh0 = a_0 g = [0.03125, 0.234375]
#   gA = [-7.375, -2.125]
# ---------------------------------------------------------------------------
DYADIC = dict(
    A=np.array([[-LN2, -2 * LN2]]),
    delta=np.array([1.0, 2.0, 1.0]).reshape(1, 3, 1),
    x=np.array([2.0, -1.0, 4.0]).reshape(1, 3, 1),
    b=np.array([[1, 2], [0.5, -1], [3, 0]], dtype=float).reshape(1, 3, 2),
    c=np.array([[1, 1], [2, 0.5], [-1, 2]], dtype=float).reshape(1, 3, 2),
    h0=np.array([4.0, -8.0]).reshape(1, 1, 2),
    dy=np.array([1.0, -2.0, 0.5]).reshape(1, 3, 1),
    dhT=np.array([1.0, -1.0]).reshape(1, 1, 2),
)


def test_dyadic_worked_example_forward():
    e = DYADIC
    y, hT, H = oracle.fwd(e["x"], e["delta"], e["A"], e["b"], e["c"], e["h0"], return_H=True)
    np.testing.assert_allclose(y.ravel(), [6.0, 1.0625, -10.9375], rtol=0, atol=1e-14)
    np.testing.assert_allclose(hT.ravel(), [12.0, 0.53125], rtol=0, atol=1e-14)
    np.testing.assert_allclose(H.reshape(3, 2), [[4, 2], [0, 2.125], [12, 0.53125]], rtol=0, atol=1e-14)


def test_dyadic_worked_example_backward():
    e = DYADIC
    gx, gd, gb, gc, gA, gh0 = oracle.bwd(e["dy"], e["x"], e["delta"], e["A"], e["b"], e["c"], e["h0"], e["dhT"])
    tol = dict(rtol=0, atol=1e-13)
    np.testing.assert_allclose(gx.ravel(), [1.9375, -1.75, 1.5], **tol)
    np.testing.assert_allclose(gd.ravel(), [3.625 * LN2 + 3.875, 4 * LN2 + 0.875, 6.0], **tol)
    np.testing.assert_allclose(gb.reshape(3, 2), [[0.125, 1.875], [7.5, 2.0], [2.0, 0.0]], **tol)
    np.testing.assert_allclose(gc.reshape(3, 2), [[4.0, 2.0], [0.0, -4.25], [6.0, 0.265625]], **tol)
    np.testing.assert_allclose(gA.ravel(), [-7.375, -2.125], **tol)
    np.testing.assert_allclose(gh0.ravel(), [0.03125, 0.234375], **tol)


# P1: delta == 0 gives a = 1 and no injection, so the state stays at h0.
def test_zero_delta_keeps_state():
    e = rand_case(2, 9, 5, 4, seed=11)
    delta = np.zeros_like(e["delta"])
    y, hT = oracle.fwd(e["x"], delta, e["A"], e["b"], e["c"], e["h0"])
    assert np.array_equal(hT, e["h0"])  # bitwise
    y_ref = np.einsum("bdn,btn->btd", e["h0"], e["c"])
    assert rel_err(y, y_ref) < 1e-15


# P2: one step, closed form.
def test_single_step_closed_form():
    e = rand_case(3, 1, 7, 8, seed=12)
    y, hT = oracle.fwd(e["x"], e["delta"], e["A"], e["b"], e["c"], e["h0"])
    dl = e["delta"][:, 0, :, None]
    h1 = np.exp(dl * e["A"][None]) * e["h0"] + dl * e["b"][:, 0, None, :] * e["x"][:, 0, :, None]
    assert rel_err(hT, h1) < 1e-15
    assert rel_err(y[:, 0], np.einsum("bdn,bn->bd", h1, e["c"][:, 0])) < 1e-15


def unrolled_forward(x, delta, A, b, c, h0):
    """h_t written out as a sum of products: each decay between steps s and t is
    exp(A * (sum of delta over (s, t])), an exponential of a SUM of steps, not the
    product of per-step exponentials the recurrence forms.  O(T^2) per (b,d,n)."""
    B, T, D = x.shape
    DS = A.shape[1]
    y = np.zeros((B, T, D))
    hT = np.zeros((B, D, DS))
    for bb in range(B):
        for d in range(D):
            for t in range(T):
                acc_y = []
                for n in range(DS):
                    An = A[d, n]
                    init = 0.0 if h0 is None else h0[bb, d, n]
                    terms = [math.exp(An * math.fsum(delta[bb, 0:t + 1, d])) * init]
                    for s in range(t + 1):
                        decay = math.exp(An * math.fsum(delta[bb, s + 1:t + 1, d]))
                        terms.append(decay * delta[bb, s, d] * b[bb, s, n] * x[bb, s, d])
                    h = math.fsum(terms)
                    acc_y.append(h * c[bb, t, n])
                    if t == T - 1:
                        hT[bb, d, n] = h
                y[bb, t, d] = math.fsum(acc_y)
    return y, hT


# P3 (DS = 1) and P4 (any DS): the unrolled sum of products.
@pytest.mark.parametrize("B,T,D,DS,h0", [(2, 12, 3, 1, True), (1, 16, 2, 4, True), (2, 10, 3, 2, False),
                                         (1, 24, 2, 16, True), (1, 7, 1, 8, True)])
def test_unrolled_sum_of_products(B, T, D, DS, h0):
    e = rand_case(B, T, D, DS, seed=100 + T + DS, h0=h0)
    y, hT = oracle.fwd(e["x"], e["delta"], e["A"], e["b"], e["c"], e["h0"])
    y_ref, hT_ref = unrolled_forward(e["x"], e["delta"], e["A"], e["b"], e["c"], e["h0"])
    assert rel_err(y, y_ref) < 1e-12
    assert rel_err(hT, hT_ref) < 1e-12


def test_unrolled_tiny_workload_shape():
    """The 1x64x16x4 workload itself (A = -(n+1), h0 = 0) against the unrolled form."""
    inp = workloads.make_inputs(workloads.get("tiny_fwd"))
    e = {k: (None if v is None else v.double().numpy()) for k, v in inp.items()}
    y, hT = oracle.fwd(e["x"], e["delta"], e["A"], e["b"], e["c"], e["h0"])
    y_ref, hT_ref = unrolled_forward(e["x"], e["delta"], e["A"], e["b"], e["c"], e["h0"])
    assert rel_err(y, y_ref) < 1e-12
    assert rel_err(hT, hT_ref) < 1e-12


# P5: with h0 = 0 the map x -> y is linear; for fixed states y is linear in c.
def test_linearity():
    e = rand_case(2, 20, 4, 4, seed=13, h0=False)
    x2 = rand_case(2, 20, 4, 4, seed=14, h0=False)["x"]
    al, be = 0.7, -1.3
    y1, _ = oracle.fwd(e["x"], e["delta"], e["A"], e["b"], e["c"])
    y2, _ = oracle.fwd(x2, e["delta"], e["A"], e["b"], e["c"])
    y12, _ = oracle.fwd(al * e["x"] + be * x2, e["delta"], e["A"], e["b"], e["c"])
    assert rel_err(y12, al * y1 + be * y2) < 1e-12
    c2 = rand_case(2, 20, 4, 4, seed=15)["c"]
    ya, _ = oracle.fwd(e["x"], e["delta"], e["A"], e["b"], c2)
    yab, _ = oracle.fwd(e["x"], e["delta"], e["A"], e["b"], al * e["c"] + be * c2)
    assert rel_err(yab, al * y1 + be * ya) < 1e-12


# P6: running [0, T1) then [T1, T) with h0 <- hT is the same computation.
def test_chunk_composition():
    e = rand_case(2, 40, 5, 8, seed=16)
    y, hT = oracle.fwd(e["x"], e["delta"], e["A"], e["b"], e["c"], e["h0"])
    h = e["h0"]
    ys = []
    for t0, t1 in [(0, 13), (13, 14), (14, 40)]:
        sl = slice(t0, t1)
        yc, h = oracle.fwd(e["x"][:, sl], e["delta"][:, sl], e["A"], e["b"][:, sl], e["c"][:, sl], h)
        ys.append(yc)
    assert np.array_equal(np.concatenate(ys, axis=1), y)
    assert np.array_equal(h, hT)


# P7: A -> -inf removes all memory: exp underflows to exactly 0, h_t = delta_t b_t x_t.
def test_memoryless_limit():
    e = rand_case(2, 15, 4, 4, seed=17)
    A = np.full_like(e["A"], -1e6)
    y, hT = oracle.fwd(e["x"], e["delta"], A, e["b"], e["c"], e["h0"])
    y_ref = e["delta"] * e["x"] * np.einsum("btn,btn->bt", e["b"], e["c"])[:, :, None]
    assert rel_err(y, y_ref) < 1e-15
    hT_ref = (e["delta"][:, -1, :, None] * e["b"][:, -1, None, :] * e["x"][:, -1, :, None])
    assert rel_err(hT, hT_ref) < 1e-15


def test_empty_sequence_passes_state_through():
    e = rand_case(2, 0, 3, 4, seed=18, dhT=True)
    y, hT = oracle.fwd(e["x"], e["delta"], e["A"], e["b"], e["c"], e["h0"])
    assert y.shape == (2, 0, 3) and np.array_equal(hT, e["h0"])
    y, hT = oracle.fwd(e["x"], e["delta"], e["A"], e["b"], e["c"], None)
    assert np.array_equal(hT, np.zeros((2, 3, 4)))
    gx, gd, gb, gc, gA, gh0 = oracle.bwd(e["dy"], e["x"], e["delta"], e["A"], e["b"], e["c"], e["h0"], e["dhT"])
    assert np.array_equal(gh0, e["dhT"]) and np.array_equal(gA, np.zeros((3, 4)))
    assert gx.shape == (2, 0, 3) and gb.shape == (2, 0, 4)


def test_thread_count_does_not_change_results():
    e = rand_case(3, 30, 37, 4, seed=19, dhT=True)
    r1 = oracle.fwd(e["x"], e["delta"], e["A"], e["b"], e["c"], e["h0"], nthreads=1)
    r5 = oracle.fwd(e["x"], e["delta"], e["A"], e["b"], e["c"], e["h0"], nthreads=5)
    for a, b in zip(r1, r5):
        assert np.array_equal(a, b)
    g1 = oracle.bwd(e["dy"], e["x"], e["delta"], e["A"], e["b"], e["c"], e["h0"], e["dhT"], nthreads=1)
    g5 = oracle.bwd(e["dy"], e["x"], e["delta"], e["A"], e["b"], e["c"], e["h0"], e["dhT"], nthreads=5)
    for a, b in zip(g1, g5):
        assert np.array_equal(a, b)


def _loss(e, **over):
    v = dict(e)
    v.update(over)
    y, hT = oracle.fwd(v["x"], v["delta"], v["A"], v["b"], v["c"], v["h0"], nthreads=1)
    return float(np.sum(e["dy"] * y) + np.sum(e["dhT"] * hT))


# P9: central finite differences of L = sum(dy*y) + sum(dhT*hT) for all six inputs.
def test_gradients_match_finite_differences():
    e = rand_case(2, 6, 3, 4, seed=20, dhT=True)
    grads = oracle.bwd(e["dy"], e["x"], e["delta"], e["A"], e["b"], e["c"], e["h0"], e["dhT"])
    names = ["x", "delta", "b", "c", "A", "h0"]
    order = {"x": 0, "delta": 1, "b": 2, "c": 3, "A": 4, "h0": 5}
    eps = 1e-6
    for nm in names:
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
        err = rel_err(grads[order[nm]], fd)
        assert err < 1e-7, (nm, err)


def _torch_plain_loop(x, delta, b, c, A, h0):
    # the plain loop the pssa_kernels.py page prints as scan_reference, transcribed into torch
    # fp64 (a one-line recurrence in broadcasting form has essentially this one shape); it is
    # a pin because the page prints it, and its gradients come from autograd, not from the
    # oracle's adjoint sweep
    T = x.shape[1]
    h = h0
    ys = []
    for t in range(T):
        h = torch.exp(delta[:, t, :, None] * A) * h + delta[:, t, :, None] * b[:, t, None, :] * x[:, t, :, None]
        ys.append((h * c[:, t, None, :]).sum(-1))
    return torch.stack(ys, 1), h


@pytest.mark.parametrize("shape", [(2, 7, 64, 16), (1, 33, 5, 4), (3, 12, 9, 2)])
def test_gradients_match_autograd_of_plain_loop(shape):
    B, T, D, DS = shape
    e = rand_case(B, T, D, DS, seed=21 + T, dhT=True)
    ts = {k: torch.tensor(e[k], dtype=torch.float64, requires_grad=True) for k in ["x", "delta", "b", "c", "A", "h0"]}
    y, hT = _torch_plain_loop(ts["x"], ts["delta"], ts["b"], ts["c"], ts["A"], ts["h0"])
    L = (torch.tensor(e["dy"]) * y).sum() + (torch.tensor(e["dhT"]) * hT).sum()
    ref = torch.autograd.grad(L, [ts[k] for k in ["x", "delta", "b", "c", "A", "h0"]])
    got = oracle.bwd(e["dy"], e["x"], e["delta"], e["A"], e["b"], e["c"], e["h0"], e["dhT"])
    for nm, g, r in zip(["gx", "gdelta", "gb", "gc", "gA", "gh0"], got, ref):
        assert rel_err(g, r.numpy()) < 1e-12, nm
    yo, hTo = oracle.fwd(e["x"], e["delta"], e["A"], e["b"], e["c"], e["h0"])
    assert rel_err(yo, y.detach().numpy()) < 1e-12


# P10: exact identities between the gradients from invariances of the map.
#  (delta, x, A) -> (l delta, x/l, A/l) leaves y, hT fixed: sum d gd = sum x gx + sum A gA
#  (x, b) -> (l x, b/l):                                    sum x gx = sum b gb
#  (b, h0, c) -> (l b, l h0, c/l): y fixed, hT scales:      sum b gb + sum h0 gh0 = sum c gc + sum dhT hT
#  (x, h0) -> (l x, l h0): everything scales:               sum x gx + sum h0 gh0 = sum dy y + sum dhT hT
def gradient_identity_residuals(e, y, hT, grads):
    gx, gd, gb, gc, gA, gh0 = grads
    s = lambda a, b: float(np.sum(np.asarray(a, np.float64) * np.asarray(b, np.float64)))
    sa = lambda a, b: float(np.sum(np.abs(np.asarray(a, np.float64) * np.asarray(b, np.float64))))
    h0 = e["h0"] if e["h0"] is not None else np.zeros_like(gh0)
    dhT = e["dhT"] if e["dhT"] is not None else np.zeros_like(gh0)
    ids = [
        (s(e["delta"], gd) - s(e["x"], gx) - s(e["A"], gA), sa(e["delta"], gd) + sa(e["x"], gx) + sa(e["A"], gA)),
        (s(e["x"], gx) - s(e["b"], gb), sa(e["x"], gx) + sa(e["b"], gb)),
        (s(e["b"], gb) + s(h0, gh0) - s(e["c"], gc) - s(dhT, hT),
         sa(e["b"], gb) + sa(h0, gh0) + sa(e["c"], gc) + sa(dhT, hT)),
        (s(e["x"], gx) + s(h0, gh0) - s(e["dy"], y) - s(dhT, hT),
         sa(e["x"], gx) + sa(h0, gh0) + sa(e["dy"], y) + sa(dhT, hT)),
    ]
    return [abs(r) / max(scale, 1e-300) for r, scale in ids]


def test_gradient_scaling_identities():
    e = rand_case(3, 64, 20, 16, seed=22, dhT=True)
    y, hT = oracle.fwd(e["x"], e["delta"], e["A"], e["b"], e["c"], e["h0"])
    grads = oracle.bwd(e["dy"], e["x"], e["delta"], e["A"], e["b"], e["c"], e["h0"], e["dhT"])
    res = gradient_identity_residuals(e, y, hT, grads)
    assert max(res) < 1e-13, res


def test_gradients_without_h0_and_dhT():
    """Absent h0 / dhT mean zeros (the pssa_kernels.py page seeds the sweep from dy alone)."""
    e = rand_case(2, 11, 6, 4, seed=23, h0=False)
    z = np.zeros((2, 6, 4))
    a = oracle.bwd(e["dy"], e["x"], e["delta"], e["A"], e["b"], e["c"], None, None)
    b = oracle.bwd(e["dy"], e["x"], e["delta"], e["A"], e["b"], e["c"], z, z)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_golden_tiny_forward_is_reproduced():
    """Regression guard: the stored oracle output for the tiny workload (written by
    tests/golden/make_golden.py) is reproduced exactly."""
    import json
    import os

    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_fwd_oracle.json")
    with open(path) as f:
        doc = json.load(f)
    inp = workloads.make_inputs(workloads.get(doc["workload"]))
    y, hT = oracle.fwd(inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"])
    assert np.array_equal(y.ravel(), np.array(doc["y"]))
    assert np.array_equal(hT.ravel(), np.array(doc["hT"]))


def test_workload_generator_is_deterministic():
    w = workloads.get("selftest")
    a = workloads.make_inputs(w)
    b = workloads.make_inputs(w)
    for k in a:
        assert (a[k] is None) == (b[k] is None)
        if a[k] is not None:
            assert torch.equal(a[k], b[k])
    assert bool((a["delta"] > 0).all()) and bool((a["A"] < 0).all())


def test_missing_required_inputs_raise_instead_of_reading_null():
    """x, delta, A, b, c (and dy for the backward) are required; a None among them raises
    before the C loops run (they would otherwise read through a NULL pointer)."""
    inp = workloads.make_inputs(workloads.custom(1, 3, 2, 2, seed=4, with_dy=True))
    args = [inp[k] for k in ("x", "delta", "A", "b", "c")]
    for i, name in enumerate(("x", "delta", "A", "b", "c")):
        bad = list(args)
        bad[i] = None
        with pytest.raises(ValueError, match=name):
            oracle.fwd(*bad)
        with pytest.raises(ValueError, match=name):
            oracle.bwd(inp["dy"], *bad)
    with pytest.raises(ValueError, match="dy"):
        oracle.bwd(None, *args)
