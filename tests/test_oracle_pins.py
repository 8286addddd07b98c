"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: hand-worked
examples (tests/golden/), a library routine (torch conv1d, torch autograd,
numpy matmul), an independent dense-matrix formulation, finite differences,
or an invariant the definition implies (causality, batch isolation, the
residual, equivalence of the two parameterisations, linearity).
Definitions: "Dynamic Short Convolutions Improve Transformers" (gist.science
Technical Summary, Methodology -> Dynamic Short Convolutions: Mechanism,
Parameterization, Placement; Efficient Training Implementation -> Fused
Low-Rank Kernel).
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch

from oracle import HEADWISE, LOWRANK, Shape
from tests import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

SHAPES = [
    Shape(B=2, T=7, d=5, D=8, k=3, kind=HEADWISE, n_heads=4),
    Shape(B=1, T=9, d=3, D=6, k=4, kind=HEADWISE, n_heads=3),
    Shape(B=2, T=6, d=4, D=5, k=2, kind=LOWRANK, rank=3),
    Shape(B=1, T=10, d=6, D=4, k=4, kind=LOWRANK, rank=2),
]
EDGE_SHAPES = [
    Shape(B=1, T=1, d=3, D=4, k=4, kind=HEADWISE, n_heads=2),   # T = 1
    Shape(B=2, T=2, d=3, D=4, k=4, kind=LOWRANK, rank=2),       # T < k
    Shape(B=1, T=5, d=2, D=3, k=1, kind=LOWRANK, rank=1),       # k = 1
    Shape(B=1, T=8, d=2, D=6, k=8, kind=HEADWISE, n_heads=6),   # k = 8, one channel per head
]


def _ids(shapes):
    return [f"{'hw' if s.kind == HEADWISE else 'lr'}-B{s.B}T{s.T}d{s.d}D{s.D}k{s.k}" for s in shapes]


# ---------------------------------------------------------------------------
# hand-worked examples
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("fname", ["worked_headwise.json", "worked_lowrank.json"])
def test_golden_worked_example(orc, fname):
    g = json.load(open(os.path.join(GOLDEN, fname)))
    sh = g["shape"]
    kind = HEADWISE if sh["kind"] == "headwise" else LOWRANK
    s = Shape(B=sh["B"], T=sh["T"], d=sh["d"], D=sh["D"], k=sh["k"], kind=kind,
              n_heads=sh.get("n_heads", 0), rank=sh.get("rank", 0))
    arr = {k: (None if g.get(k) is None else np.array(g[k], dtype=np.float64))
           for k in ("h", "x", "dy", "W", "A", "U", "w0")}
    fw = orc.forward(s, arr["h"], arr["x"], W=arr["W"], A=arr["A"], U=arr["U"], w0=arr["w0"])
    bw = orc.backward(s, arr["h"], arr["x"], arr["dy"], W=arr["W"], A=arr["A"], U=arr["U"],
                      w0=arr["w0"])
    got = {"y": fw["y"], **bw}
    for key, want in g["expect"].items():
        np.testing.assert_allclose(got[key], np.array(want, dtype=np.float64), rtol=0, atol=1e-12,
                                   err_msg=key)


# ---------------------------------------------------------------------------
# static special case: zero generator -> static depthwise conv with w0
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("s", SHAPES + EDGE_SHAPES, ids=_ids(SHAPES + EDGE_SHAPES))
def test_zero_generator_is_static_conv(orc, s):
    rng = np.random.default_rng(1)
    p = pins.random_problem(rng, s)
    for key in ("W", "A"):
        if p.get(key) is not None:
            p[key] = np.zeros_like(p[key])
    fw = orc.forward(s, p["h"], p["x"], **pins.gen_args(p))
    x = torch.tensor(p["x"]).reshape(s.B, s.T, s.D)
    w0 = torch.tensor(p["w0"], requires_grad=True)
    xt = x.clone().requires_grad_(True)
    ref = pins.static_conv_torch(xt, w0)
    np.testing.assert_allclose(fw["y"] - p["x"], ref.detach().reshape(-1, s.D).numpy(),
                               rtol=1e-12, atol=1e-12)
    # backward of the static case: dx and dw0 from torch autograd of conv1d
    dy = torch.tensor(p["dy"]).reshape(s.B, s.T, s.D)
    ((ref + xt) * dy).sum().backward()
    bw = orc.backward(s, p["h"], p["x"], p["dy"], **pins.gen_args(p))
    np.testing.assert_allclose(bw["dx"], xt.grad.reshape(-1, s.D).numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(bw["dw0"], w0.grad.numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("s", SHAPES, ids=_ids(SHAPES))
def test_zero_filter_is_identity(orc, s):
    """No generator and no bias: y == x and dx == dy exactly (the residual)."""
    rng = np.random.default_rng(2)
    p = pins.random_problem(rng, s, bias=False)
    for key in ("W", "U"):
        if p.get(key) is not None:
            p[key] = np.zeros_like(p[key])
    fw = orc.forward(s, p["h"], p["x"], **pins.gen_args(p))
    assert np.array_equal(fw["y"], p["x"])
    bw = orc.backward(s, p["h"], p["x"], p["dy"], **pins.gen_args(p))
    assert np.array_equal(bw["dx"], p["dy"])


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("s", SHAPES, ids=_ids(SHAPES))
def test_causality(orc, s):
    """Perturbing x and h after t leaves y up to t bitwise unchanged."""
    rng = np.random.default_rng(3)
    p = pins.random_problem(rng, s)
    y0 = orc.forward(s, p["h"], p["x"], **pins.gen_args(p))["y"].reshape(s.B, s.T, s.D)
    for t in range(s.T - 1):
        q = dict(p)
        x = p["x"].reshape(s.B, s.T, s.D).copy()
        h = p["h"].reshape(s.B, s.T, s.d).copy()
        x[:, t + 1:] += rng.standard_normal(x[:, t + 1:].shape)
        h[:, t + 1:] += rng.standard_normal(h[:, t + 1:].shape)
        q["x"], q["h"] = x.reshape(-1, s.D), h.reshape(-1, s.d)
        y1 = orc.forward(s, q["h"], q["x"], **pins.gen_args(q))["y"].reshape(s.B, s.T, s.D)
        assert np.array_equal(y0[:, : t + 1], y1[:, : t + 1]), t
        assert not np.array_equal(y0[:, t + 1:], y1[:, t + 1:])


@pytest.mark.parametrize("s", [sh for sh in SHAPES if sh.B > 1], ids=_ids([sh for sh in SHAPES if sh.B > 1]))
def test_batch_isolation(orc, s):
    rng = np.random.default_rng(4)
    p = pins.random_problem(rng, s)
    y0 = orc.forward(s, p["h"], p["x"], **pins.gen_args(p))["y"].reshape(s.B, s.T, s.D)
    x = p["x"].reshape(s.B, s.T, s.D).copy()
    h = p["h"].reshape(s.B, s.T, s.d).copy()
    x[1] += 1.0
    h[1] -= 1.0
    y1 = orc.forward(s, h.reshape(-1, s.d), x.reshape(-1, s.D), **pins.gen_args(p))["y"]
    y1 = y1.reshape(s.B, s.T, s.D)
    assert np.array_equal(y0[0], y1[0])
    assert not np.array_equal(y0[1], y1[1])


@pytest.mark.parametrize("s", SHAPES + EDGE_SHAPES, ids=_ids(SHAPES + EDGE_SHAPES))
def test_dense_matrix_form(orc, s):
    """Per channel, y_c = (I + M_c) x_c and dx_c = (I + M_c)^T dy_c."""
    rng = np.random.default_rng(5)
    p = pins.random_problem(rng, s)
    fw = orc.forward(s, p["h"], p["x"], **pins.gen_args(p))
    bw = orc.backward(s, p["h"], p["x"], p["dy"], **pins.gen_args(p))
    w = fw["w"]
    for b in range(s.B):
        rows = slice(b * s.T, (b + 1) * s.T)
        for c in range(s.D):
            M = np.eye(s.T) + pins.dense_conv_matrix(w, b, c, s.T)
            np.testing.assert_allclose(fw["y"][rows, c], M @ p["x"][rows, c], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(bw["dx"][rows, c], M.T @ p["dy"][rows, c], rtol=1e-12,
                                       atol=1e-12)


@pytest.mark.parametrize("s", SHAPES + EDGE_SHAPES, ids=_ids(SHAPES + EDGE_SHAPES))
def test_generator_is_matmul(orc, s):
    """Step 1 equals a library matmul; step 2 matches the tying / product rule."""
    rng = np.random.default_rng(6)
    p = pins.random_problem(rng, s)
    w, gen = orc.filters(s, p["h"], **pins.gen_args(p))
    if s.kind == HEADWISE:
        u = p["h"] @ p["W"]
        np.testing.assert_allclose(gen, u, rtol=1e-12, atol=1e-12)
        hd = s.D // s.n_heads
        for c in range(s.D):
            np.testing.assert_allclose(w[:, c, :] - p["w0"][c],
                                       u[:, (c // hd) * s.k:(c // hd + 1) * s.k], rtol=1e-12, atol=1e-12)
    else:
        z = p["h"] @ p["A"]
        np.testing.assert_allclose(gen, z, rtol=1e-12, atol=1e-12)
        v = (z @ p["U"]).reshape(-1, s.D, s.k)
        np.testing.assert_allclose(w - p["w0"][None], v, rtol=1e-12, atol=1e-12)


def test_headwise_equals_lowrank(orc):
    """Head-wise (n_h, W) == low-rank with r = d, A = I, U[i, c*k+j] = W[i, head(c)*k+j]."""
    rng = np.random.default_rng(7)
    sh = Shape(B=2, T=6, d=3, D=6, k=3, kind=HEADWISE, n_heads=2)
    sl = Shape(B=2, T=6, d=3, D=6, k=3, kind=LOWRANK, rank=3)
    p = pins.random_problem(rng, sh)
    hd = sh.D // sh.n_heads
    U = np.zeros((3, sh.D * sh.k))
    for c in range(sh.D):
        U[:, c * sh.k:(c + 1) * sh.k] = p["W"][:, (c // hd) * sh.k:(c // hd + 1) * sh.k]
    A = np.eye(3)
    fh = orc.forward(sh, p["h"], p["x"], W=p["W"], w0=p["w0"])
    fl = orc.forward(sl, p["h"], p["x"], A=A, U=U, w0=p["w0"])
    np.testing.assert_allclose(fh["y"], fl["y"], rtol=1e-12, atol=1e-12)
    bh = orc.backward(sh, p["h"], p["x"], p["dy"], W=p["W"], w0=p["w0"])
    bl = orc.backward(sl, p["h"], p["x"], p["dy"], A=A, U=U, w0=p["w0"])
    for key in ("dx", "dh", "dw0"):
        np.testing.assert_allclose(bh[key], bl[key], rtol=1e-12, atol=1e-12, err_msg=key)
    dW_from_dU = np.zeros_like(bh["dW"])
    for c in range(sh.D):
        e = c // hd
        dW_from_dU[:, e * sh.k:(e + 1) * sh.k] += bl["dU"][:, c * sh.k:(c + 1) * sh.k]
    np.testing.assert_allclose(bh["dW"], dW_from_dU, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("s", [EDGE_SHAPES[2]], ids=_ids([EDGE_SHAPES[2]]))
def test_k1_closed_form(orc, s):
    """k = 1: y = x * (1 + w[..., 0]) elementwise."""
    rng = np.random.default_rng(8)
    p = pins.random_problem(rng, s)
    fw = orc.forward(s, p["h"], p["x"], **pins.gen_args(p))
    np.testing.assert_allclose(fw["y"], p["x"] * (1.0 + fw["w"][..., 0]), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("s", SHAPES[:2] + SHAPES[2:3], ids=_ids(SHAPES[:2] + SHAPES[2:3]))
def test_linearity(orc, s):
    """y - x is linear in x at fixed h, and linear in the generator weights + bias."""
    rng = np.random.default_rng(9)
    p = pins.random_problem(rng, s)
    q = pins.random_problem(rng, s)
    a, b = 0.75, -1.25
    f = lambda x: orc.forward(s, p["h"], x, **pins.gen_args(p))["y"] - x
    np.testing.assert_allclose(f(a * p["x"] + b * q["x"]), a * f(p["x"]) + b * f(q["x"]),
                               rtol=1e-11, atol=1e-11)
    if s.kind == HEADWISE:
        g = lambda W, w0: orc.forward(s, p["h"], p["x"], W=W, w0=w0)["y"] - p["x"]
        np.testing.assert_allclose(g(a * p["W"] + b * q["W"], a * p["w0"] + b * q["w0"]),
                                   a * g(p["W"], p["w0"]) + b * g(q["W"], q["w0"]),
                                   rtol=1e-11, atol=1e-11)
    else:
        g = lambda U, w0: orc.forward(s, p["h"], p["x"], A=p["A"], U=U, w0=w0)["y"] - p["x"]
        np.testing.assert_allclose(g(a * p["U"] + b * q["U"], a * p["w0"] + b * q["w0"]),
                                   a * g(p["U"], p["w0"]) + b * g(q["U"], q["w0"]),
                                   rtol=1e-11, atol=1e-11)


# ---------------------------------------------------------------------------
# gradients
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("s", SHAPES + EDGE_SHAPES, ids=_ids(SHAPES + EDGE_SHAPES))
def test_grads_match_torch_autograd(orc, s):
    rng = np.random.default_rng(10)
    p = pins.random_problem(rng, s)
    ref = pins.torch_grads(s, p)
    bw = orc.backward(s, p["h"], p["x"], p["dy"], **pins.gen_args(p))
    names = {"x": "dx", "h": "dh", "w0": "dw0", "W": "dW", "A": "dA", "U": "dU"}
    for leaf, g in ref.items():
        got = bw[names[leaf]].reshape(g.shape)
        np.testing.assert_allclose(got, g, rtol=1e-11, atol=1e-11, err_msg=leaf)


@pytest.mark.parametrize("s", SHAPES[:1] + SHAPES[2:3] + EDGE_SHAPES[1:2],
                         ids=_ids(SHAPES[:1] + SHAPES[2:3] + EDGE_SHAPES[1:2]))
def test_grads_central_differences(orc, s):
    """Central differences of L = sum(dy*y) on every coordinate of every input."""
    rng = np.random.default_rng(11)
    p = pins.random_problem(rng, s)
    bw = orc.backward(s, p["h"], p["x"], p["dy"], **pins.gen_args(p))
    names = {"x": "dx", "h": "dh", "w0": "dw0", "W": "dW", "A": "dA", "U": "dU"}
    eps = 1e-3
    for leaf, gname in names.items():
        if p.get(leaf) is None:
            continue
        base = p[leaf]
        num = np.zeros(base.size)
        for i in range(base.size):
            for sign in (+1, -1):
                q = dict(p)
                arr = base.copy().reshape(-1)
                arr[i] += sign * eps
                q[leaf] = arr.reshape(base.shape)
                num[i] += sign * pins.loss(orc, s, q)
        num /= 2 * eps
        np.testing.assert_allclose(bw[gname].reshape(-1), num, rtol=1e-7, atol=1e-7, err_msg=leaf)


@pytest.mark.parametrize("s", SHAPES, ids=_ids(SHAPES))
def test_adjoint_identity(orc, s):
    """L is affine in each input alone, so L(p + delta) - L(p) = <grad, delta> exactly."""
    rng = np.random.default_rng(12)
    p = pins.random_problem(rng, s)
    bw = orc.backward(s, p["h"], p["x"], p["dy"], **pins.gen_args(p))
    names = {"x": "dx", "h": "dh", "w0": "dw0", "W": "dW", "A": "dA", "U": "dU"}
    L0 = pins.loss(orc, s, p)
    for leaf, gname in names.items():
        if p.get(leaf) is None:
            continue
        delta = rng.standard_normal(p[leaf].shape)
        q = dict(p)
        q[leaf] = p[leaf] + delta
        lhs = pins.loss(orc, s, q) - L0
        rhs = float((bw[gname].reshape(delta.shape) * delta).sum())
        assert abs(lhs - rhs) <= 1e-9 * max(1.0, abs(rhs)), (leaf, lhs, rhs)


# ---------------------------------------------------------------------------
# packed documents: a row holding several documents back to back is the
# documents run alone (the window never reaches across a document start)
# ---------------------------------------------------------------------------
PACKED = [
    # (shape with T unset, document lengths): lengths below k, of one token,
    # and an empty document
    (Shape(B=1, T=0, d=5, D=8, k=4, kind=HEADWISE, n_heads=4), (1, 6, 2, 3, 9)),
    (Shape(B=1, T=0, d=4, D=6, k=3, kind=LOWRANK, rank=3), (5, 1, 1, 7, 4)),
    (Shape(B=1, T=0, d=3, D=4, k=8, kind=HEADWISE, n_heads=2), (10, 3, 0, 8)),
]


def _packed_shape(base: Shape, lens) -> Shape:
    from dataclasses import replace
    cu = tuple(int(c) for c in np.cumsum((0,) + tuple(lens)))
    return replace(base, T=cu[-1], cu_seqlens=cu)


GRADS = ("dW", "dA", "dU", "dw0")


@pytest.mark.parametrize("base,lens", PACKED, ids=[f"{'hw' if b.kind == HEADWISE else 'lr'}-{l}" for b, l in PACKED])
def test_packed_equals_documents_run_alone(orc, base, lens):
    """Per-token outputs (y, the generator values, dx, dh) of the packed row
    equal bitwise those of each document run as its own sequence; the weight
    gradients are the sums of the documents' (up to summation order)."""
    from dataclasses import replace
    s = _packed_shape(base, lens)
    rng = np.random.default_rng(21)
    p = pins.random_problem(rng, s)
    fw = orc.forward(s, p["h"], p["x"], **pins.gen_args(p))
    bw = orc.backward(s, p["h"], p["x"], p["dy"], **pins.gen_args(p))
    total = {g: None for g in GRADS}
    t0 = 0
    for L in lens:
        if L == 0:
            continue
        sd = replace(base, T=L)
        q = {k: (None if v is None else (v[t0:t0 + L] if k in ("h", "x", "dy") else v)) for k, v in p.items()}
        fd = orc.forward(sd, q["h"], q["x"], **pins.gen_args(q))
        bd = orc.backward(sd, q["h"], q["x"], q["dy"], **pins.gen_args(q))
        assert np.array_equal(np.asarray(fw["y"])[t0:t0 + L], np.asarray(fd["y"]))
        assert np.array_equal(np.asarray(fw["gen"])[t0:t0 + L], np.asarray(fd["gen"]))
        for key in ("dx", "dh"):
            assert np.array_equal(np.asarray(bw[key])[t0:t0 + L], np.asarray(bd[key])), key
        for g in GRADS:
            if bd.get(g) is not None:
                total[g] = bd[g] if total[g] is None else total[g] + bd[g]
        t0 += L
    for g in GRADS:
        if total[g] is not None:
            np.testing.assert_allclose(bw[g], total[g], rtol=1e-12, atol=1e-12, err_msg=g)


@pytest.mark.parametrize("s", SHAPES[1:2] + SHAPES[3:4], ids=_ids(SHAPES[1:2] + SHAPES[3:4]))
def test_one_document_is_the_plain_row(orc, s):
    """A single document covering the row changes nothing, bitwise."""
    from dataclasses import replace
    rng = np.random.default_rng(22)
    p = pins.random_problem(rng, s)
    sp = replace(s, cu_seqlens=(0, s.B * s.T))
    for a, b in ((orc.forward(s, p["h"], p["x"], **pins.gen_args(p)),
                  orc.forward(sp, p["h"], p["x"], **pins.gen_args(p))),
                 (orc.backward(s, p["h"], p["x"], p["dy"], **pins.gen_args(p)),
                  orc.backward(sp, p["h"], p["x"], p["dy"], **pins.gen_args(p)))):
        for key in a:
            if a[key] is not None:
                assert np.array_equal(np.asarray(a[key]), np.asarray(b[key])), key


@pytest.mark.parametrize("s", [sh for sh in SHAPES if sh.B > 1], ids=_ids([sh for sh in SHAPES if sh.B > 1]))
def test_equal_documents_are_the_batch(orc, s):
    """B documents of length T packed into one row equal the [B, T] batch
    bitwise, weight gradients included (same token order in every sum)."""
    from dataclasses import replace
    rng = np.random.default_rng(23)
    p = pins.random_problem(rng, s)
    sp = replace(s, B=1, T=s.B * s.T, cu_seqlens=tuple(range(0, s.B * s.T + 1, s.T)))
    a = {**orc.forward(s, p["h"], p["x"], **pins.gen_args(p)),
         **orc.backward(s, p["h"], p["x"], p["dy"], **pins.gen_args(p))}
    b = {**orc.forward(sp, p["h"], p["x"], **pins.gen_args(p)),
         **orc.backward(sp, p["h"], p["x"], p["dy"], **pins.gen_args(p))}
    for key in a:
        if a[key] is not None:
            assert np.array_equal(np.asarray(a[key]).reshape(-1), np.asarray(b[key]).reshape(-1)), key


# ---------------------------------------------------------------------------
# the producing projection x = h Wp (the layer's input, from the same h)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("s", SHAPES + EDGE_SHAPES[:2], ids=_ids(SHAPES + EDGE_SHAPES[:2]))
def test_proj_is_matmul(orc, s):
    """x = h Wp equals a numpy matmul, and a unit column of Wp copies a column of h."""
    rng = np.random.default_rng(24)
    h = rng.standard_normal((s.B * s.T, s.d))
    Wp = rng.standard_normal((s.d, s.D))
    np.testing.assert_allclose(orc.proj(s, h, Wp), h @ Wp, rtol=1e-13, atol=1e-13)
    E = np.zeros((s.d, s.D))
    for c in range(s.D):
        E[c % s.d, c] = 1.0
    assert np.array_equal(orc.proj(s, h, E), h[:, [c % s.d for c in range(s.D)]])
