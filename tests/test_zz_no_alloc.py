"""dynconv_fwd_noalloc (the forward whose workspace is the library's static
per-GPU scratch) against dynconv_fwd with a caller workspace: same kernels,
so y and the generator cache must be bitwise equal.  Two calls in a row, the
second on a smaller input, so the second runs on scratch that still holds
the first call's contents.  A call that needs more than the scratch holds is
refused and leaves its outputs untouched."""
from __future__ import annotations

import sys

import pytest
import torch

import input_dependent_depthwise_amd as dc
import workloads
from tests import gpu_util as gu
from workloads import HEADWISE, LOWRANK, Workload

pytestmark = pytest.mark.gpu

PAIRS = [
    # (first call, second smaller call)
    (Workload("na_hw_bf16_big", B=2, T=2048, d=512, D=1088, k=4, kind=HEADWISE, n_heads=16, seed=61),
     Workload("na_hw_bf16_small", B=1, T=300, d=512, D=1088, k=4, kind=HEADWISE, n_heads=16, seed=62)),
    (Workload("na_lr_bf16_big", B=4, T=1024, d=768, D=2304, k=4, kind=LOWRANK, rank=16, seed=63),
     Workload("na_lr_bf16_small", B=2, T=129, d=768, D=2304, k=4, kind=LOWRANK, rank=16, seed=64)),
    (Workload("na_hw_bf16_wide_big", B=1, T=4096, d=256, D=4352, k=4, kind=HEADWISE, n_heads=64, seed=65),
     Workload("na_lr_bf16_r32_small", B=1, T=77, d=256, D=512, k=3, kind=LOWRANK, rank=32, seed=66)),
    (Workload("na_lr_fp32_big", B=2, T=500, d=64, D=128, k=4, kind=LOWRANK, rank=8, dtype="fp32", seed=67),
     Workload("na_hw_fp32_small", B=1, T=33, d=32, D=48, k=3, kind=HEADWISE, n_heads=3, dtype="fp32", seed=68)),
]


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _kw(w, dev):
    return dict(k=w.k, W=dev.get("W"), A=dev.get("A"), U=dev.get("U"), w0=dev.get("w0"), n_heads=w.n_heads)


def _check_one(w, dev, with_cache):
    kw = _kw(w, dev)
    if with_cache:
        y_ref, c_ref = dc.dynconv_fwd(dev["h"], dev["x"], want_cache=True, **kw)
        cache = torch.full_like(c_ref, float("nan"))
        y = torch.full_like(dev["x"], float("nan"))
        dc.dynconv_fwd_noalloc(dev["h"], dev["x"], y=y, gen_cache=cache, **kw)
        torch.cuda.synchronize()
        assert torch.equal(cache, c_ref), w.name
    else:
        y_ref = dc.dynconv_fwd(dev["h"], dev["x"], **kw)
        y = torch.full_like(dev["x"], float("nan"))
        dc.dynconv_fwd_noalloc(dev["h"], dev["x"], y=y, **kw)
        torch.cuda.synchronize()
    assert torch.equal(y, y_ref), (w.name, with_cache)
    return y


@pytest.mark.parametrize("pair", PAIRS, ids=[p[0].name for p in PAIRS])
@pytest.mark.parametrize("with_cache", [True, False], ids=["cache", "nocache"])
def test_noalloc_matches_fwd_two_calls(pair, with_cache):
    first, second = pair
    for w in (first, second):
        _note(f"[noalloc] {w.name} B={w.B} T={w.T} d={w.d} D={w.D} k={w.k} {w.kind} {w.dtype} cache={with_cache}")
        inp = workloads.generate(w)
        dev = gu.to_dev(inp)
        y = _check_one(w, dev, with_cache)
        # and within the parity bar of the oracle, like the forward it equals
        if w.tokens <= 4096:
            ref = gu.oracle_run(w, inp)
            gu.compare(w, {"y": y}, ref, keys=["y"])


def test_noalloc_refuses_oversized_call():
    """The Mamba-2 input-conv shape without a caller cache needs a 32 MiB
    cache slot, more than the 16 MiB scratch: refused, y untouched.  With a
    cache it fits and matches dynconv_fwd."""
    w = workloads.WORKLOADS["mamba2_inconv_headwise"]
    _note(f"[noalloc] refuse {w.name}")
    dev = gu.to_dev(workloads.generate(w, with_dy=False))
    kw = _kw(w, dev)
    y = torch.full_like(dev["x"], 3.0)
    with pytest.raises(dc.DynConvError) as e:
        dc.dynconv_fwd_noalloc(dev["h"], dev["x"], y=y, **kw)
    assert e.value.status == dc.DYNCONV_E_SCRATCH
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())
    _check_one(w, dev, with_cache=True)
    del dev
    torch.cuda.empty_cache()
