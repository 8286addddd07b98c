"""Helpers for the GPU parity tests: run the HIP path through the C ABI,
run the oracle on the same seeded inputs, compare per tensor."""
from __future__ import annotations

import numpy as np
import torch

import input_dependent_depthwise_amd as dc
import oracle
import workloads
from workloads import HEADWISE, Workload

# max relative error (normwise: max|gpu - oracle| / max|oracle|) per output
TOL = {"fp32": 1e-5, "bf16": 2e-2}


def oracle_shape(w: Workload, cu_seqlens=None) -> oracle.Shape:
    return oracle.Shape(B=w.B, T=w.T, d=w.d, D=w.D, k=w.k,
                        kind=oracle.HEADWISE if w.kind == HEADWISE else oracle.LOWRANK,
                        n_heads=w.n_heads, rank=w.rank,
                        cu_seqlens=None if cu_seqlens is None else tuple(int(c) for c in cu_seqlens))


def to_dev(inp: dict, device="cuda") -> dict:
    return {k: (None if v is None else v.to(device).contiguous()) for k, v in inp.items()}


def gpu_run(w: Workload, dev_inp: dict, use_cache: bool = True, need_dh: bool = True,
            need_dw0: bool = True, fwd_cache: bool = True, cu_seqlens=None):
    """Forward + backward on the GPU; returns dict of device tensors.

    fwd_cache=False runs the forward without a caller cache (the library keeps
    the generator values in its workspace); the backward then recomputes it.
    cu_seqlens (a list of document offsets): the single row holds packed
    documents.
    """
    kw = dict(k=w.k, W=dev_inp.get("W"), A=dev_inp.get("A"), U=dev_inp.get("U"),
              w0=dev_inp.get("w0"), n_heads=w.n_heads)
    if cu_seqlens is not None:
        kw["cu_seqlens"] = torch.tensor(list(cu_seqlens), dtype=torch.int32, device=dev_inp["x"].device)
    if fwd_cache:
        y, cache = dc.dynconv_fwd(dev_inp["h"], dev_inp["x"], want_cache=True, **kw)
    else:
        y, cache = dc.dynconv_fwd(dev_inp["h"], dev_inp["x"], **kw), None
    g = dc.dynconv_bwd(dev_inp["h"], dev_inp["x"], dev_inp["dy"], gen_cache=cache if use_cache else None,
                       need_dh=need_dh, need_dw0=need_dw0 and dev_inp.get("w0") is not None, **kw)
    torch.cuda.synchronize()
    return {"y": y, "cache": cache, **g}


def oracle_run(w: Workload, inp: dict, cu_seqlens=None) -> dict:
    s = oracle_shape(w, cu_seqlens)
    args = dict(W=inp.get("W"), A=inp.get("A"), U=inp.get("U"), w0=inp.get("w0"))
    fw = oracle.forward(s, inp["h"], inp["x"], **args)
    bw = oracle.backward(s, inp["h"], inp["x"], inp["dy"], w=fw["w"], **args)
    out = {"y": fw["y"], "cache": fw["gen"], **bw}
    del fw
    return out


def max_rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64).reshape(-1)
    ref = np.asarray(ref, dtype=np.float64).reshape(-1)
    assert got.shape == ref.shape
    scale = np.abs(ref).max() if ref.size else 0.0
    err = np.abs(got - ref).max() if ref.size else 0.0
    if scale == 0.0:
        return float(err)
    return float(err / scale)


def compare(w: Workload, gpu: dict, ref: dict, keys=None) -> dict:
    """Per-tensor max relative error; asserts each is within TOL[w.dtype]."""
    tol = TOL[w.dtype]
    keys = keys or [k for k in ("y", "dx", "dh", "dw0", "dW", "dA", "dU", "cache") if k in gpu and k in ref
                    and gpu[k] is not None]
    errs = {}
    for k in keys:
        g = gpu[k].detach().float().cpu().numpy()
        errs[k] = max_rel_err(g, ref[k])
    bad = {k: e for k, e in errs.items() if not (e <= tol)}
    assert not bad, f"{w.name}: max relative error above {tol}: {bad} (all: {errs})"
    return errs
