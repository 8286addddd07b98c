"""The static filter (generator kind DYNCONV_STATIC: w[t,c,j] = w0[c,j], no
generator) on the GPU against the fp64 oracle.

The oracle has no separate static routine: the static filter is its
head-wise layer with a zero generator (one head, W = 0, h = 0), which its pins
tie to torch's conv1d.  Covers the vector fast paths (ring forward, backward
without generator sums), the per-element paths (D = 100, fp32), k = 1 and
k = 5..8, packed documents, the decode step, the fused producing projection,
dh filled with zeros, and the autograd wrapper.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import input_dependent_depthwise_amd as dc
import oracle
import workloads
from tests import gpu_util as gu
from workloads import HEADWISE, Workload

pytestmark = pytest.mark.gpu


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _w(name, B, T, D, k, dtype="bf16", seed=0):
    # one head over all channels; d_model 1 for the oracle's zero generator
    return Workload(name, B=B, T=T, d=1, D=D, k=k, kind=HEADWISE, n_heads=1, dtype=dtype, seed=seed)


STATIC = [
    _w("st_bf16_k4", 2, 300, 512, 4, seed=601),
    _w("st_bf16_k3_D4352", 2, 2048, 4352, 3, seed=602),
    _w("st_bf16_k1", 3, 70, 256, 1, seed=603),
    _w("st_bf16_k2_T1", 3, 1, 128, 2, seed=604),
    _w("st_bf16_k8", 2, 150, 256, 8, seed=605),
    _w("st_bf16_k6_D100", 2, 75, 100, 6, seed=606),
    _w("st_bf16_D100", 2, 75, 100, 4, seed=607),
    _w("st_fp32_k5", 2, 100, 48, 5, dtype="fp32", seed=608),
    _w("st_fp32_k4", 2, 100, 64, 4, dtype="fp32", seed=609),
]


def _inputs(w):
    inp = workloads.generate(w)
    if inp["w0"] is None:
        raise AssertionError("the static filter needs w0")
    return inp


def _oracle(w, inp, cu_seqlens=None):
    s = gu.oracle_shape(w, cu_seqlens)
    h0 = torch.zeros(w.B, w.T, 1, dtype=torch.float64)
    W0 = torch.zeros(1, w.k, dtype=torch.float64)
    fw = oracle.forward(s, h0, inp["x"], W=W0, w0=inp["w0"])
    bw = oracle.backward(s, h0, inp["x"], inp["dy"], W=W0, w0=inp["w0"], w=fw["w"])
    return {"y": fw["y"], "dx": bw["dx"], "dw0": bw["dw0"]}


def _gpu(w, inp, cu_seqlens=None, h=None):
    dev = gu.to_dev(inp)
    kw = dict(k=w.k, w0=dev["w0"])
    if cu_seqlens is not None:
        kw["cu_seqlens"] = torch.tensor(cu_seqlens, dtype=torch.int32, device="cuda")
    y = dc.dynconv_fwd(h, dev["x"], **kw)
    g = dc.dynconv_bwd(h, dev["x"], dev["dy"], **kw)
    torch.cuda.synchronize()
    return {"y": y, **g}


@pytest.mark.parametrize("w", STATIC, ids=[w.name for w in STATIC])
def test_static_parity(w):
    _note(f"[static] {w.name} B={w.B} T={w.T} D={w.D} k={w.k} {w.dtype}")
    inp = _inputs(w)
    got = _gpu(w, inp)
    errs = gu.compare(w, got, _oracle(w, inp), keys=["y", "dx", "dw0"])
    _note(f"[static] {w.name} errors {errs}")


def test_static_packed():
    w = _w("st_pk", 1, 308, 512, 4, seed=610)
    cu = [int(c) for c in np.cumsum((0, 1, 2, 3, 70, 0, 5, 130, 33, 64))]
    inp = _inputs(w)
    gu.compare(w, _gpu(w, inp, cu), _oracle(w, inp, cu), keys=["y", "dx", "dw0"])


def test_static_dh_is_zero_and_generator_free():
    """With h given, dh comes back as zeros (y does not depend on h), and the
    results equal the call without h bitwise."""
    w = STATIC[0]
    inp = _inputs(w)
    h = torch.randn(w.B, w.T, 64, device="cuda").to(torch.bfloat16)
    a = _gpu(w, inp, h=h)
    b = _gpu(w, inp)
    assert torch.count_nonzero(a["dh"]) == 0
    for k in ("y", "dx", "dw0"):
        assert torch.equal(a[k], b[k]), k


def test_static_decode():
    """Decode steps with the static filter equal the forward's rows."""
    w = _w("st_dec", 5, 12, 256, 4, seed=611)
    inp = _inputs(w)
    dev = gu.to_dev(inp)
    y_full = dc.dynconv_fwd(None, dev["x"], k=w.k, w0=dev["w0"])
    state = torch.zeros(w.B, w.k - 1, w.D, dtype=torch.bfloat16, device="cuda")
    for t in range(w.T):
        yt = dc.dynconv_decode(None, dev["x"][:, t].clone(), state, k=w.k, w0=dev["w0"])
        torch.cuda.synchronize()
        assert gu.max_rel_err(yt.float().cpu().numpy(), y_full[:, t].float().cpu().numpy()) < 1e-2, t


def test_static_autograd():
    w = STATIC[0]
    inp = _inputs(w)
    dev = gu.to_dev(inp)
    ref = _gpu(w, inp)
    x = dev["x"].clone().requires_grad_(True)
    w0 = dev["w0"].clone().requires_grad_(True)
    y = dc.DynConvFn.apply(None, x, None, None, None, w0, w.k, 0)
    y.backward(dev["dy"])
    torch.cuda.synchronize()
    assert torch.equal(y.detach(), ref["y"])
    assert torch.equal(x.grad, ref["dx"])
    assert gu.max_rel_err(w0.grad.float().cpu().numpy(), ref["dw0"].float().cpu().numpy()) < 1e-2


def test_static_with_projection():
    """dynconv_fwd_proj with the static filter: x = h Wp, then the static conv."""
    w = Workload("st_proj", B=2, T=200, d=128, D=512, k=4, kind=HEADWISE, n_heads=1, seed=612)
    inp = _inputs(w)
    Wp = workloads.generate_proj_weight(w)
    dev = gu.to_dev(inp)
    x, y = dc.dynconv_fwd_proj(dev["h"], Wp.cuda(), k=w.k, w0=dev["w0"])
    torch.cuda.synchronize()
    s = gu.oracle_shape(w)
    xr = oracle.proj(s, inp["h"], Wp)
    assert gu.max_rel_err(x.float().cpu().numpy(), xr) < 2e-2
    wz = w.with_(d=1)
    ref = oracle.forward(gu.oracle_shape(wz), torch.zeros(w.B, w.T, 1, dtype=torch.float64), x.cpu(),
                         W=torch.zeros(1, w.k, dtype=torch.float64), w0=inp["w0"])
    assert gu.max_rel_err(y.float().cpu().numpy(), ref["y"]) < 2e-2
