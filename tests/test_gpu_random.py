"""GPU parity on seeded random shapes: the HIP path (through the C ABI)
against the fp64 oracle, element by element, on 300 training-step problems
drawn from a fixed generator, and 80 decode runs, 80 fused-projection
forwards and 40 static-filter steps drawn the same way.

The draw covers the combinations the hand-picked cases take one at a time:
both generator kinds, fp32 and bf16 I/O, 1 to 8 taps, ranks 1 to 64, head
widths from 1 to 136 channels (aligned to 8-channel vectors, straddling them,
4 mod 8), widths D and d_model that are and are not whole 16-byte vectors,
sequence lengths around the 32-token tiles (1, 2, k - 1, 31..33, 63..65,
127..129, ...), batches of 1 to 3, with and without the bias, with the
forward's cache passed on, recomputed by the backward, or kept in the
forward's workspace, and single rows of packed documents of random lengths
(empty documents and documents shorter than the filter included).  Each
problem is small enough for the oracle to finish in well under a second.

Tolerance: the same max relative error per output tensor as every other
parity case (1e-5 for fp32 I/O, 2e-2 for bf16 I/O).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import workloads
from tests import gpu_util as gu
from workloads import HEADWISE, LOWRANK, Workload

N_CASES = 300
T_CHOICES = [1, 2, 3, 5, 7, 17, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 200, 257, 300, 511, 520]
HD_CHOICES = [1, 2, 3, 4, 5, 6, 7, 8, 10, 12, 16, 20, 24, 28, 32, 36, 40, 60, 64, 68, 72, 96, 100, 128, 132, 136]


def _draw(i: int):
    """Problem i of the sweep: (workload, how the cache is handled, document offsets or None)."""
    r = np.random.RandomState(1000 + i)
    dtype = "fp32" if r.rand() < 0.15 else "bf16"
    kind = HEADWISE if r.rand() < 0.5 else LOWRANK
    k = int(r.choice([1, 2, 3, 4, 4, 4, 3, 5, 6, 7, 8]))
    packed = r.rand() < 0.2
    B = 1 if packed else int(r.randint(1, 4))
    T = int(r.choice(T_CHOICES))
    d = int(8 * r.randint(1, 41)) if r.rand() < 0.75 else int(r.randint(1, 300))
    n_heads = rank = 0
    if kind == HEADWISE:
        hd = int(r.choice(HD_CHOICES))
        max_heads = max(1, min(256 // k, 2200 // hd))
        n_heads = int(r.randint(1, max_heads + 1))
        D = n_heads * hd
    else:
        rank = int(r.randint(1, 65))
        D = int(8 * r.randint(1, 260)) if r.rand() < 0.8 else int(r.randint(1, 2100))
    # keep the oracle's work small: tokens x channels and tokens x d_model x generator columns
    N = n_heads * k if kind == HEADWISE else rank
    while T > 1 and (B * T * D > 1_200_000 or B * T * d * N > 60_000_000):
        T = max(1, T // 2)
    bias_std = 0.1 if r.rand() < 0.8 else 0.0
    x_dist = "silu_gated" if r.rand() < 0.2 else "normal"
    mode = str(r.choice(["reuse", "reuse", "recompute", "ws_cache"]))
    cu = None
    if packed:
        cuts = np.sort(r.randint(0, T + 1, size=int(r.randint(0, 6))))
        cu = [0] + [int(c) for c in cuts] + [T]
    w = Workload(f"rand{i:03d}", B=B, T=T, d=d, D=D, k=k, kind=kind, n_heads=n_heads, rank=rank, dtype=dtype,
                 seed=5000 + i, bias_std=bias_std, x_dist=x_dist)
    return w, mode, cu


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES))
def test_random_parity(i):
    w, mode, cu = _draw(i)
    print(f"[random] {w.name} B={w.B} T={w.T} d={w.d} D={w.D} k={w.k} {w.kind} heads={w.n_heads} "
          f"rank={w.rank} {w.dtype} bias={w.bias_std > 0} cache={mode} docs={cu}", flush=True)
    sys.stdout.flush()
    inp = workloads.generate(w)
    got = gu.gpu_run(w, gu.to_dev(inp), use_cache=mode == "reuse", fwd_cache=mode != "ws_cache", cu_seqlens=cu)
    ref = gu.oracle_run(w, inp, cu_seqlens=cu)
    errs = gu.compare(w, got, ref)
    print(f"[random] {w.name} errors {errs}", flush=True)


def test_random_draw_is_valid():
    """Every drawn problem satisfies the boundary's shape rules (host only)."""
    for i in range(N_CASES):
        w, mode, cu = _draw(i)
        assert w.D > 0 and w.d > 0 and 1 <= w.k <= 8 and w.T >= 1
        if w.kind == HEADWISE:
            assert w.D % w.n_heads == 0 and w.n_heads * w.k <= 256
        else:
            assert 1 <= w.rank <= 64
        if cu is not None:
            assert w.B == 1 and cu[0] == 0 and cu[-1] == w.T and all(a <= b for a, b in zip(cu, cu[1:]))


N_DECODE = 80
N_PROJ = 80


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_DECODE))
def test_random_decode(i):
    """dynconv_decode from a zeroed history, one call per position, against
    the oracle's forward rows (up to 24 positions), on the sweep's
    one-row-per-sequence problems; the history then holds the last k-1 rows
    of x bitwise."""
    import torch

    import input_dependent_depthwise_amd as dc
    import oracle

    w, _, _ = _draw(2000 + i)
    w = w.with_(name=f"rdec{i:03d}", T=min(w.T, 24))
    print(f"[random decode] {w.name} B={w.B} T={w.T} d={w.d} D={w.D} k={w.k} {w.kind} heads={w.n_heads} "
          f"rank={w.rank} {w.dtype} bias={w.bias_std > 0}", flush=True)
    inp = workloads.generate(w, with_dy=False)
    ref = oracle.forward(gu.oracle_shape(w), inp["h"], inp["x"], W=inp.get("W"), A=inp.get("A"), U=inp.get("U"),
                         w0=inp.get("w0"))["y"]
    dev = gu.to_dev(inp)
    B, T, D = dev["x"].shape
    state = torch.zeros(B, w.k - 1, D, dtype=dev["x"].dtype, device="cuda") if w.k > 1 else None
    kw = dict(k=w.k, W=dev.get("W"), A=dev.get("A"), U=dev.get("U"), w0=dev.get("w0"), n_heads=w.n_heads)
    ys = [dc.dynconv_decode(dev["h"][:, t].clone(), dev["x"][:, t].clone(), state, **kw) for t in range(T)]
    torch.cuda.synchronize()
    err = gu.max_rel_err(torch.stack(ys, 1).float().cpu().numpy(), np.asarray(ref).reshape(B, T, D))
    assert err <= gu.TOL[w.dtype], (w.name, err)
    if w.k > 1:
        last = dev["x"][:, max(0, T - (w.k - 1)):T]
        assert torch.equal(state[:, state.shape[1] - last.shape[1]:], last)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_PROJ))
def test_random_proj(i):
    """dynconv_fwd_proj: x = h Wp against the oracle's projection (normwise
    and within the output rounding per element), y against the oracle's
    forward on the x the GPU wrote, the cache against the oracle's generator
    values; packed rows included."""
    import oracle
    from tests import test_gpu_proj as tp

    w, _, cu = _draw(3000 + i)
    w = w.with_(name=f"rproj{i:03d}")
    print(f"[random proj] {w.name} B={w.B} T={w.T} d={w.d} D={w.D} k={w.k} {w.kind} heads={w.n_heads} "
          f"rank={w.rank} {w.dtype} docs={cu}", flush=True)
    inp, Wp, x, y, cache = tp._run(w, cu)
    s = gu.oracle_shape(w, cu)
    tp._check_x(w, x, oracle.proj(s, inp["h"], Wp))
    ref = oracle.forward(s, inp["h"], x.cpu(), W=inp.get("W"), A=inp.get("A"), U=inp.get("U"), w0=inp.get("w0"))
    gu.compare(w, {"y": y, "cache": cache}, {"y": ref["y"], "cache": ref["gen"]})


N_STATIC = 40


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_STATIC))
def test_random_static(i):
    """The static filter (no generator, w = w0) on the sweep's widths, taps,
    lengths, batches and packed rows, against the oracle's head-wise layer
    with a zero generator."""
    from tests import test_gpu_static as ts

    w, _, cu = _draw(4000 + i)
    w = ts._w(f"rstat{i:03d}", w.B, w.T, w.D, w.k, dtype=w.dtype, seed=7000 + i)
    print(f"[random static] {w.name} B={w.B} T={w.T} D={w.D} k={w.k} {w.dtype} docs={cu}", flush=True)
    inp = ts._inputs(w)
    got = ts._gpu(w, inp, cu)
    gu.compare(w, got, ts._oracle(w, inp, cu), keys=["y", "dx", "dw0"])
