"""GPU parity of the fused producing projection (dynconv_fwd_proj): the
layer's input x = h Wp computed from the same hidden state as the filters,
then the layer on it, against the fp64 oracle.

x is checked against the oracle's projection (normwise and per element: the
bf16 rounding of an fp32 sum), y against the oracle's forward on the x the
GPU wrote (the layer's own parity is covered elsewhere), the generator cache
against the oracle's generator values.  Shapes cover the fused matrix-core
path (D, N and d_model multiples of 8, bf16), ragged row blocks, a d_model
tail, and the plain fallbacks (N, D or d_model not a multiple of 8, fp32);
the full-size workloads are checked on sampled rows and whole sequence-start
windows.
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
from workloads import HEADWISE, LOWRANK, WORKLOADS, Workload

pytestmark = pytest.mark.gpu


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


PROJ = [
    # fused: matrix-core GEMM against [Wp | W] or [Wp | A]
    Workload("pj_hw_bf16_N16_ragged", B=2, T=300, d=128, D=512, k=4, kind=HEADWISE, n_heads=4, seed=91),
    Workload("pj_hw_bf16_N256_d200", B=1, T=333, d=200, D=512, k=4, kind=HEADWISE, n_heads=64, seed=92),
    Workload("pj_hw_bf16_hd68", B=2, T=130, d=96, D=544, k=4, kind=HEADWISE, n_heads=8, seed=93),
    Workload("pj_lr_bf16_r16", B=2, T=300, d=128, D=384, k=4, kind=LOWRANK, rank=16, seed=94),
    Workload("pj_lr_bf16_r32_k3", B=1, T=200, d=256, D=1024, k=3, kind=LOWRANK, rank=32, seed=95,
             bias_std=0.0),
    Workload("pj_hw_bf16_T1", B=3, T=1, d=32, D=64, k=4, kind=HEADWISE, n_heads=4, seed=96),
    # plain fallbacks
    Workload("pj_lr_bf16_r5_N5", B=2, T=97, d=40, D=200, k=2, kind=LOWRANK, rank=5, seed=97),
    Workload("pj_hw_bf16_D100", B=2, T=75, d=64, D=100, k=4, kind=HEADWISE, n_heads=4, seed=98),
    Workload("pj_lr_bf16_d60", B=2, T=80, d=60, D=128, k=4, kind=LOWRANK, rank=16, seed=99),
    Workload("pj_hw_fp32_k5", B=2, T=100, d=32, D=48, k=5, kind=HEADWISE, n_heads=3, dtype="fp32", seed=100),
    Workload("pj_lr_bf16_r1_k1", B=2, T=64, d=32, D=64, k=1, kind=LOWRANK, rank=1, seed=101),
]


def _gen_args(w, dev):
    return dict(W=dev.get("W"), A=dev.get("A"), U=dev.get("U"), w0=dev.get("w0"), n_heads=w.n_heads)


def _f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _check_x(w, x_gpu, x_ref):
    """x: normwise within the bf16 tolerance, and per element within the
    rounding of the output (half an ulp, 2^-9 relative for bf16) plus the
    fp32 accumulation's error, taken as 1e-4 of the largest |x|."""
    g = _f64(x_gpu).reshape(x_ref.shape)
    err = gu.max_rel_err(g, x_ref)
    assert err <= gu.TOL[w.dtype], f"x normwise {err}"
    ulp = 2.0 ** -8 if w.dtype == "bf16" else 2.0 ** -23
    bound = ulp * np.abs(x_ref) + 1e-4 * np.abs(x_ref).max()
    bad = np.abs(g - x_ref) > bound
    assert not bad.any(), f"x: {int(bad.sum())} elements beyond the rounding bound"
    return err


def _run(w, cu_seqlens=None):
    inp = workloads.generate(w, with_dy=False)
    Wp = workloads.generate_proj_weight(w)
    dev = gu.to_dev(inp)
    kw = {}
    if cu_seqlens is not None:
        kw["cu_seqlens"] = torch.tensor(cu_seqlens, dtype=torch.int32, device="cuda")
    x, y, cache = dc.dynconv_fwd_proj(dev["h"], Wp.cuda(), k=w.k, want_cache=True, **_gen_args(w, dev), **kw)
    torch.cuda.synchronize()
    return inp, Wp, x, y, cache


@pytest.mark.parametrize("w", PROJ, ids=[w.name for w in PROJ])
def test_proj_parity(w):
    _note(f"[proj] {w.name} B={w.B} T={w.T} d={w.d} D={w.D} k={w.k} {w.kind} N={w.gen_cols} {w.dtype}")
    inp, Wp, x, y, cache = _run(w)
    s = gu.oracle_shape(w)
    ex = _check_x(w, x, oracle.proj(s, inp["h"], Wp))
    ref = oracle.forward(s, inp["h"], x.cpu(), W=inp.get("W"), A=inp.get("A"), U=inp.get("U"), w0=inp.get("w0"))
    errs = gu.compare(w, {"y": y, "cache": cache}, {"y": ref["y"], "cache": ref["gen"]})
    _note(f"[proj] {w.name} x {ex:.3g} {errs}")


def test_proj_packed():
    """Packed documents: the projection is per token; the layer on the
    projected x follows the document table."""
    w = PROJ[2].with_(name="pj_pk_hd68", B=1, T=308)
    lens = (1, 2, 3, 70, 0, 5, 130, 33, 64)
    cu = [int(c) for c in np.cumsum((0,) + lens)]
    inp, Wp, x, y, cache = _run(w, cu)
    s = gu.oracle_shape(w, cu)
    _check_x(w, x, oracle.proj(s, inp["h"], Wp))
    ref = oracle.forward(s, inp["h"], x.cpu(), W=inp["W"], w0=inp["w0"])
    gu.compare(w, {"y": y, "cache": cache}, {"y": ref["y"], "cache": ref["gen"]})


def test_proj_matches_separate_calls():
    """The fused call's y and cache agree with dynconv_fwd on the x it wrote
    (the generator values differ only by fp32 summation order)."""
    w = PROJ[0]
    inp, Wp, x, y, cache = _run(w)
    dev = gu.to_dev(inp)
    y2, cache2 = dc.dynconv_fwd(dev["h"], x, k=w.k, want_cache=True, **_gen_args(w, dev))
    torch.cuda.synchronize()
    assert gu.max_rel_err(_f64(cache), _f64(cache2)) < 1e-5
    assert gu.max_rel_err(_f64(y), _f64(y2)) < 1e-2


@pytest.mark.parametrize("name", [n for n, w in WORKLOADS.items() if w.dtype == "bf16"])
def test_proj_full_workload(name):
    """Full size, the shapes the benchmark times: x on 64 sampled rows, y and
    the cache on the first 128 tokens of every sequence (windows that start
    at a sequence start, so the oracle sees the same history), and y against
    dynconv_fwd on the same x."""
    w = WORKLOADS[name]
    _note(f"[proj full] {name}")
    inp, Wp, x, y, cache = _run(w)
    rng = np.random.default_rng(5)
    rows = np.sort(rng.choice(w.tokens, size=64, replace=False))
    h2 = inp["h"].reshape(w.tokens, w.d)
    s1 = gu.oracle_shape(w.with_(B=1, T=64))
    _check_x(w, x.reshape(w.tokens, w.D)[torch.as_tensor(rows, device="cuda")], oracle.proj(s1, h2[rows], Wp))
    L = 128
    sw = gu.oracle_shape(w.with_(T=L))
    ref = oracle.forward(sw, inp["h"][:, :L], x[:, :L].cpu(), W=inp.get("W"), A=inp.get("A"), U=inp.get("U"),
                         w0=inp.get("w0"))
    gu.compare(w, {"y": y[:, :L], "cache": cache.reshape(w.B, w.T, -1)[:, :L]},
               {"y": ref["y"], "cache": ref["gen"]})
    dev = gu.to_dev(inp)
    y2, cache2 = dc.dynconv_fwd(dev["h"], x, k=w.k, want_cache=True, **_gen_args(w, dev))
    torch.cuda.synchronize()
    ec, ey = gu.max_rel_err(_f64(cache), _f64(cache2)), gu.max_rel_err(_f64(y), _f64(y2))
    _note(f"[proj full] {name} vs separate calls: cache {ec:.3g} y {ey:.3g} "
          f"bitwise={torch.equal(cache, cache2) and torch.equal(y, y2)}")
    assert ec < 1e-5 and ey < 1e-2
    del dev, x, y, cache, y2, cache2
    torch.cuda.empty_cache()
