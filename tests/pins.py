"""Independent formulations the oracle is pinned against (test code only).

None of these calls the oracle; each computes some part of the layer by a
route other than the oracle's loops, so that a mistake in the oracle (a
dropped term, a wrong sign or index, a transposed operand) shows up as a
disagreement.  Definitions follow "Dynamic Short Convolutions Improve
Transformers" (gist.science Technical Summary, Methodology -> Dynamic Short
Convolutions: Mechanism, Parameterization, Placement).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from oracle import HEADWISE, LOWRANK, Shape


def random_problem(rng: np.random.Generator, s: Shape, bias: bool = True, scale: float = 0.5):
    """fp64 random inputs for shape ``s`` (numpy)."""
    p = {
        "h": rng.standard_normal((s.B * s.T, s.d)),
        "x": rng.standard_normal((s.B * s.T, s.D)),
        "dy": rng.standard_normal((s.B * s.T, s.D)),
        "w0": scale * rng.standard_normal((s.D, s.k)) if bias else None,
    }
    if s.kind == HEADWISE:
        p["W"] = scale * rng.standard_normal((s.d, s.n_heads * s.k))
    else:
        p["A"] = scale * rng.standard_normal((s.d, s.rank))
        p["U"] = scale * rng.standard_normal((s.rank, s.D * s.k))
    return p


def gen_args(p):
    return {k: p.get(k) for k in ("W", "A", "U", "w0")}


def static_conv_torch(x_btd: torch.Tensor, w0: torch.Tensor) -> torch.Tensor:
    """Causal depthwise conv with a fixed per-channel filter, via torch conv1d.

    conv1d is a cross-correlation: out[t] = sum_m weight[m] * in[t + m - pad].
    With left padding k-1 and weight[c, 0, m] = w0[c, k-1-m], out[t] =
    sum_j w0[c, j] x[t-j], i.e. tap j is the lag j.
    """
    B, T, D = x_btd.shape
    k = w0.shape[1]
    weight = torch.flip(w0, dims=[1]).reshape(D, 1, k)
    xin = torch.nn.functional.pad(x_btd.transpose(1, 2), (k - 1, 0))
    return torch.nn.functional.conv1d(xin, weight, groups=D).transpose(1, 2)


def dense_conv_matrix(w_btdk: np.ndarray, b: int, c: int, T: int) -> np.ndarray:
    """M_c[t, s] = w_t[c, t-s] for 0 <= t-s < k: the conv as a T x T matrix."""
    k = w_btdk.shape[-1]
    M = np.zeros((T, T))
    for t in range(T):
        for j in range(k):
            if t - j >= 0:
                M[t, t - j] = w_btdk[b * T + t, c, j]
    return M


def torch_forward(s: Shape, h, x, W=None, A=None, U=None, w0=None):
    """The forward written with torch tensor ops (shifts, einsum-free matmuls)."""
    B, T, D, k = s.B, s.T, s.D, s.k
    h = h.reshape(B, T, s.d)
    x = x.reshape(B, T, D)
    if s.kind == HEADWISE:
        hd = D // s.n_heads
        u = (h @ W).reshape(B, T, s.n_heads, 1, k)
        w = u.expand(B, T, s.n_heads, hd, k).reshape(B, T, D, k)
    else:
        z = h @ A
        w = (z @ U).reshape(B, T, D, k)
    if w0 is not None:
        w = w + w0.reshape(1, 1, D, k)
    y = x.clone()
    for j in range(k):
        if j >= T:
            break
        shifted = torch.cat([torch.zeros(B, j, D, dtype=x.dtype), x[:, : T - j]], dim=1)
        y = y + w[..., j] * shifted
    return y.reshape(B * T, D)


def torch_grads(s: Shape, p):
    """Gradients of L = sum(dy * y) by torch autograd of ``torch_forward``."""
    leaves = {}
    for key in ("h", "x", "W", "A", "U", "w0"):
        if p.get(key) is not None:
            leaves[key] = torch.tensor(p[key], dtype=torch.float64, requires_grad=True)
    y = torch_forward(s, leaves["h"], leaves["x"], W=leaves.get("W"), A=leaves.get("A"),
                      U=leaves.get("U"), w0=leaves.get("w0"))
    L = (y * torch.tensor(p["dy"], dtype=torch.float64)).sum()
    L.backward()
    return {k: v.grad.numpy() for k, v in leaves.items()}


def loss(orc: "oracle.OracleLib", s: Shape, p) -> float:
    y = orc.forward(s, p["h"], p["x"], **gen_args(p))["y"]
    return float((y * p["dy"]).sum())
