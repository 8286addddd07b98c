"""HIP graph capture of the library's calls (through torch.cuda.graph).

The library enqueues kernels only (no allocation, copy, memset or
synchronisation), so a training step or a run of decoding steps can be
captured once and replayed.  Each test captures the calls on static input
tensors, then, several times, writes new inputs into those tensors, replays
the graph, synchronises, runs the same calls eagerly on the same inputs and
checks that every output of the replay equals the eager result bitwise (the
kernels are deterministic, so replay and eager run take the same summation
order).  One replay is also checked against the fp64 oracle.
"""
from __future__ import annotations

import sys

import pytest
import torch

import input_dependent_depthwise_amd as dc
import workloads
from tests import gpu_util as gu
from workloads import HEADWISE, LOWRANK, Workload

pytestmark = pytest.mark.gpu

CASES = [
    Workload("gr_hw_bf16_hd68", B=2, T=300, d=128, D=544, k=4, kind=HEADWISE, n_heads=8, seed=301),
    Workload("gr_lr_bf16_r16", B=2, T=257, d=128, D=384, k=4, kind=LOWRANK, rank=16, seed=302),
    Workload("gr_lr_fp32_r8_k3", B=2, T=100, d=32, D=64, k=3, kind=LOWRANK, rank=8, dtype="fp32", seed=303),
]
REPLAYS = 3


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _step(w, t):
    kw = dict(k=w.k, W=t.get("W"), A=t.get("A"), U=t.get("U"), w0=t.get("w0"), n_heads=w.n_heads)
    y, cache = dc.dynconv_fwd(t["h"], t["x"], want_cache=True, **kw)
    g = dc.dynconv_bwd(t["h"], t["x"], t["dy"], gen_cache=cache, need_dh=True, need_dw0=True, **kw)
    return {"y": y, "cache": cache, **g}


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_graph_replay_training_step(w):
    _note(f"[graph] {w.name}")
    static = gu.to_dev(workloads.generate(w))
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):  # warm-up outside the capture
        _step(w, static)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = _step(w, static)
    for r in range(REPLAYS):
        fresh = workloads.generate(w.with_(seed=w.seed + 100 + r))
        for key, v in fresh.items():
            if v is not None:
                static[key].copy_(v.to("cuda"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        eager = _step(w, static)
        torch.cuda.synchronize()
        for key, v in eager.items():
            if v is not None:
                assert torch.equal(out[key], v), (w.name, r, key)
        if r == REPLAYS - 1:
            gu.compare(w, {k: v for k, v in out.items()}, gu.oracle_run(w, fresh))
        _note(f"[graph] {w.name} replay {r} equals the eager step")


def test_graph_replay_decode():
    """Eight decoding steps captured once (the history updated in place by
    each step), replayed on new tokens; y and the history equal an eager run
    from the same history."""
    w = Workload("gr_dec_hw", B=4, T=8, d=64, D=512, k=4, kind=HEADWISE, n_heads=8, seed=304)
    _note(f"[graph] {w.name}")
    inp = gu.to_dev(workloads.generate(w, with_dy=False))
    B, T, D = inp["x"].shape
    kw = dict(k=w.k, W=inp["W"], w0=inp["w0"], n_heads=w.n_heads)
    hs = [inp["h"][:, t].clone() for t in range(T)]
    xs = [inp["x"][:, t].clone() for t in range(T)]
    state = torch.zeros(B, w.k - 1, D, dtype=inp["x"].dtype, device="cuda")
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        dc.dynconv_decode(hs[0], xs[0], state.clone(), **kw)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ys = [dc.dynconv_decode(hs[t], xs[t], state, **kw) for t in range(T)]
    gen = torch.Generator().manual_seed(7)
    for r in range(REPLAYS):
        for t in range(T):
            hs[t].copy_(torch.randn(hs[t].shape, generator=gen).to(hs[t]))
            xs[t].copy_(torch.randn(xs[t].shape, generator=gen).to(xs[t]))
        start = torch.randn(state.shape, generator=gen).to(state)
        state.copy_(start)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        st2 = start.clone()
        ref = [dc.dynconv_decode(hs[t], xs[t], st2, **kw) for t in range(T)]
        torch.cuda.synchronize()
        for t in range(T):
            assert torch.equal(ys[t], ref[t]), (r, t)
        assert torch.equal(state, st2), r
        _note(f"[graph] {w.name} replay {r} equals the eager steps")
