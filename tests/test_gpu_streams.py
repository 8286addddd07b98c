"""Concurrent calls: the library keeps no device state between calls (every
pass works in its caller's workspace), so independent problems enqueued on
two streams, from two host threads, give the results of the same calls run
one after the other, bitwise."""
from __future__ import annotations

import threading

import pytest
import torch

import input_dependent_depthwise_amd as dc
import workloads
from workloads import HEADWISE, LOWRANK, Workload

pytestmark = pytest.mark.gpu

PAIR = [
    Workload("cs_hw_bf16_hd68", B=2, T=1000, d=128, D=544, k=4, kind=HEADWISE, n_heads=8, seed=311),
    Workload("cs_lr_bf16_r16", B=2, T=777, d=128, D=384, k=3, kind=LOWRANK, rank=16, seed=312),
]


def _step(w, t, stream):
    kw = dict(k=w.k, W=t.get("W"), A=t.get("A"), U=t.get("U"), w0=t.get("w0"), n_heads=w.n_heads)
    with torch.cuda.stream(stream):
        y, cache = dc.dynconv_fwd(t["h"], t["x"], want_cache=True, **kw)
        g = dc.dynconv_bwd(t["h"], t["x"], t["dy"], gen_cache=cache, need_dh=True, need_dw0=True, **kw)
    return {"y": y, "cache": cache, **g}


def test_two_streams_two_threads():
    ins = [{k: (None if v is None else v.cuda()) for k, v in workloads.generate(w).items()} for w in PAIR]
    s0 = torch.cuda.current_stream()
    ref = [_step(w, t, s0) for w, t in zip(PAIR, ins)]
    torch.cuda.synchronize()
    for rep in range(3):
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        for st in streams:
            st.wait_stream(s0)
        out = [None, None]
        errs = []

        def run(i):
            try:
                for _ in range(2):  # several calls per thread, interleaved with the other's
                    out[i] = _step(PAIR[i], ins[i], streams[i])
            except Exception as e:  # surfaced below
                errs.append(e)

        th = [threading.Thread(target=run, args=(i,)) for i in range(2)]
        for t in th:
            t.start()
        for t in th:
            t.join()
        torch.cuda.synchronize()
        assert not errs, errs
        for i in range(2):
            for key, v in ref[i].items():
                if v is not None:
                    assert torch.equal(out[i][key], v), (PAIR[i].name, rep, key)
