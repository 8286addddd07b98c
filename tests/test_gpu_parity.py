"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerance (max relative error, max|gpu - oracle| / max|oracle| per output
tensor): 1e-5 for fp32 I/O, 2e-2 for bf16 I/O with fp32 accumulation.
Covers the five workloads at their full sizes (the launch configuration the
benchmark times), shapes that span several tiles with ragged tails, and the
degenerate cases (T = 1, T < k, k = 1, heads narrower than a vector, rank 1,
no bias).  Bitwise invariants: zero filter gives y == x and dx == dy,
causality, batch isolation, determinism, cache reuse == recompute, the
autograd wrapper == the direct calls.
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


SMALL = [
    Workload("hw_bf16_hd72_ragged", B=2, T=300, d=128, D=360, k=4, kind=HEADWISE, n_heads=5, seed=11),
    Workload("hw_bf16_hd128_k3", B=1, T=257, d=64, D=1024, k=3, kind=HEADWISE, n_heads=8, seed=12),
    Workload("hw_bf16_hd68", B=2, T=130, d=96, D=544, k=4, kind=HEADWISE, n_heads=8, seed=13),
    Workload("hw_bf16_hd8_k2", B=3, T=70, d=32, D=128, k=2, kind=HEADWISE, n_heads=16, seed=14),
    Workload("hw_bf16_hd4", B=1, T=90, d=16, D=64, k=4, kind=HEADWISE, n_heads=16, seed=15),
    Workload("hw_bf16_k8_nobias", B=2, T=50, d=48, D=256, k=8, kind=HEADWISE, n_heads=4, seed=16,
             bias_std=0.0),
    Workload("hw_fp32_k5", B=2, T=100, d=32, D=48, k=5, kind=HEADWISE, n_heads=3, dtype="fp32", seed=17),
    Workload("lr_bf16_r16_ragged", B=2, T=300, d=128, D=360, k=4, kind=LOWRANK, rank=16, seed=21),
    Workload("lr_bf16_r32_k3", B=1, T=200, d=256, D=1024, k=3, kind=LOWRANK, rank=32, seed=22,
             x_dist="silu_gated"),
    Workload("lr_bf16_r1_k1", B=2, T=64, d=32, D=64, k=1, kind=LOWRANK, rank=1, seed=23),
    Workload("lr_bf16_r64_k8", B=1, T=150, d=64, D=256, k=8, kind=LOWRANK, rank=64, seed=24),
    Workload("lr_bf16_r5_k2_nobias", B=2, T=97, d=40, D=200, k=2, kind=LOWRANK, rank=5, seed=25,
             bias_std=0.0),
    Workload("lr_fp32_r8", B=2, T=77, d=32, D=64, k=4, kind=LOWRANK, rank=8, dtype="fp32", seed=26),
    Workload("hw_bf16_T1", B=3, T=1, d=32, D=64, k=4, kind=HEADWISE, n_heads=4, seed=27),
    Workload("lr_bf16_T3_lt_k", B=2, T=3, d=32, D=64, k=4, kind=LOWRANK, rank=16, seed=28),
    Workload("lr_fp32_T2", B=4, T=2, d=8, D=8, k=3, kind=LOWRANK, rank=3, dtype="fp32", seed=29),
    # head widths that are not a multiple of 8 (a 16-byte channel vector straddles two heads)
    Workload("hw_bf16_hd12_k1", B=2, T=77, d=32, D=96, k=1, kind=HEADWISE, n_heads=8, seed=31),
    Workload("hw_bf16_hd20_k3", B=1, T=129, d=48, D=160, k=3, kind=HEADWISE, n_heads=8, seed=32),
    Workload("hw_bf16_hd36_k2_nobias", B=2, T=65, d=32, D=144, k=2, kind=HEADWISE, n_heads=4, seed=33,
             bias_std=0.0),
    # rank past one 16-row block (two dz / dU blocks)
    Workload("lr_bf16_r20_k3", B=1, T=200, d=256, D=1024, k=3, kind=LOWRANK, rank=20, seed=34),
    # sequence length a multiple of the 32-token tile (the backward's halo rows
    # across a sequence start are cut at load time), several sequences
    Workload("lr_bf16_r16_T96", B=3, T=96, d=64, D=192, k=4, kind=LOWRANK, rank=16, seed=35),
    Workload("lr_bf16_r32_k3_T64", B=3, T=64, d=64, D=256, k=3, kind=LOWRANK, rank=32, seed=36),
    # widths that are not whole 16-byte vectors (plain per-element kernels)
    Workload("hw_bf16_D100", B=2, T=75, d=64, D=100, k=4, kind=HEADWISE, n_heads=4, seed=51),
    Workload("lr_bf16_D100", B=2, T=75, d=64, D=100, k=3, kind=LOWRANK, rank=16, seed=52),
    Workload("hw_fp32_D66", B=2, T=60, d=32, D=66, k=4, kind=HEADWISE, n_heads=6, dtype="fp32", seed=53),
    Workload("lr_fp32_D66_d30", B=1, T=50, d=30, D=66, k=2, kind=LOWRANK, rank=4, dtype="fp32", seed=54),
    Workload("lr_bf16_d60", B=2, T=80, d=60, D=128, k=4, kind=LOWRANK, rank=16, seed=55),
    Workload("hw_bf16_d60", B=2, T=80, d=60, D=256, k=4, kind=HEADWISE, n_heads=4, seed=56),
    # wide generator weights read in place (n_heads*k a multiple of 8, 64..256 columns): a
    # K tail (d_model 200, 136), ragged row blocks, columns padded to the 32-column tile (72)
    Workload("hw_bf16_N256_ragged", B=1, T=333, d=200, D=512, k=4, kind=HEADWISE, n_heads=64, seed=57),
    Workload("hw_bf16_N72", B=2, T=150, d=136, D=1152, k=4, kind=HEADWISE, n_heads=18, seed=58),
    # 5..8 taps on the tuned head-wise kernels (4 channels per lane in the
    # backward): straddling heads (68, 12), heads of 4 channels, a ragged
    # sequence, and a slice of the 2B QKV shape that spans many blocks
    Workload("hw_bf16_k5_hd68", B=2, T=130, d=96, D=544, k=5, kind=HEADWISE, n_heads=8, seed=41),
    Workload("hw_bf16_k6_hd12", B=1, T=200, d=32, D=96, k=6, kind=HEADWISE, n_heads=8, seed=42),
    Workload("hw_bf16_k7_hd4", B=2, T=77, d=16, D=64, k=7, kind=HEADWISE, n_heads=16, seed=43),
    Workload("hw_bf16_k8_hd128_ragged", B=2, T=333, d=64, D=1024, k=8, kind=HEADWISE, n_heads=8, seed=44),
    Workload("hw_bf16_k6_2b_slice", B=1, T=4096, d=128, D=3072, k=6, kind=HEADWISE, n_heads=24, seed=45),
    # 5..8 taps on the matrix-core low-rank kernels (a second tap half in the
    # forward; one wave per SIMD in the backward): ranks 1 .. 32, bias and no
    # bias, a slice of the 150M QKV shape
    Workload("lr_bf16_r16_k5", B=2, T=300, d=128, D=384, k=5, kind=LOWRANK, rank=16, seed=46),
    Workload("lr_bf16_r32_k8", B=1, T=200, d=256, D=1024, k=8, kind=LOWRANK, rank=32, seed=47),
    Workload("lr_bf16_r8_k6_T64", B=3, T=64, d=64, D=256, k=6, kind=LOWRANK, rank=8, seed=48, bias_std=0.0),
    Workload("lr_bf16_r20_k7", B=1, T=200, d=256, D=512, k=7, kind=LOWRANK, rank=20, seed=49),
    Workload("lr_bf16_r1_k5", B=2, T=64, d=32, D=64, k=5, kind=LOWRANK, rank=1, seed=50),
    Workload("lr_bf16_k8_150m_slice", B=2, T=2048, d=768, D=2304, k=8, kind=LOWRANK, rank=16, seed=61),
    # more wide weights: 96 and 160 columns with d_model tails (200, 136)
    Workload("hw_bf16_N96_d200", B=2, T=333, d=200, D=768, k=4, kind=HEADWISE, n_heads=24, seed=59),
    Workload("hw_bf16_N160_d136", B=1, T=200, d=136, D=1280, k=4, kind=HEADWISE, n_heads=40, seed=60),
    # wide weights on several token ranges of the generator-gradient kernels:
    # 144 columns, d_model 264 (a partial 128-row chunk), 6 taps, ragged T
    Workload("hw_bf16_N144_k6_d264", B=2, T=700, d=264, D=576, k=6, kind=HEADWISE, n_heads=24, seed=62),
    # 200 generator columns on the 256-column projection tile (a zero column
    # tail), d_model 136 (a partial 32-k step), 50 heads of 8
    Workload("hw_bf16_N200_d136", B=2, T=150, d=136, D=400, k=4, kind=HEADWISE, n_heads=50, seed=63),
    # the head-wise forward folds the batch in the last channel group when at
    # most half a wave of channels is left there and the batch holds an even
    # number of sequences: four sequences (the halves pair sequence 0 with 2
    # and 1 with 3), 128-channel heads with 16 lanes left, 24-channel heads
    # with 2 lanes left
    Workload("hw_bf16_hd68_fold_B4", B=4, T=130, d=96, D=544, k=4, kind=HEADWISE, n_heads=8, seed=64),
    Workload("hw_bf16_hd128_fold", B=2, T=211, d=64, D=640, k=4, kind=HEADWISE, n_heads=5, seed=65),
    Workload("hw_bf16_hd24_fold_k3", B=2, T=150, d=64, D=528, k=3, kind=HEADWISE, n_heads=22, seed=66),
    # folded groups with sequences shorter than the filter: one token each
    # (four sequences), and three tokens with 4 taps
    Workload("hw_bf16_fold_T1_B4", B=4, T=1, d=32, D=96, k=4, kind=HEADWISE, n_heads=8, seed=70),
    Workload("hw_bf16_fold_T3_hd68", B=2, T=3, d=32, D=544, k=4, kind=HEADWISE, n_heads=8, seed=71),
    # quad heads (4 mod 8 channels) with 4 taps and more than 128 generator
    # columns: the backward conv writes the heads within one span straight
    # into g and only the heads across span boundaries go through partials
    # (64 heads of 68 as in the Mamba-2 input conv; 40 heads of 68 with a
    # partial last span; 36 heads of 132)
    Workload("hw_bf16_hd68_N256", B=2, T=200, d=64, D=4352, k=4, kind=HEADWISE, n_heads=64, seed=67),
    Workload("hw_bf16_hd68_N160", B=1, T=333, d=96, D=2720, k=4, kind=HEADWISE, n_heads=40, seed=68),
    Workload("hw_bf16_hd132_N144", B=2, T=150, d=72, D=4752, k=4, kind=HEADWISE, n_heads=36, seed=69),
]
_BY_NAME = {w.name: w for w in SMALL}


def _run_and_compare(w: Workload, use_cache=True):
    _note(f"[parity] {w.name} B={w.B} T={w.T} d={w.d} D={w.D} k={w.k} {w.kind} "
          f"n_heads={w.n_heads} rank={w.rank} {w.dtype} cache={use_cache}")
    inp = workloads.generate(w)
    dev = gu.to_dev(inp)
    got = gu.gpu_run(w, dev, use_cache=use_cache)
    del dev
    ref = gu.oracle_run(w, inp)
    errs = gu.compare(w, got, ref)
    _note(f"[parity] {w.name} errors {errs}")
    return errs


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_parity_small(w):
    _run_and_compare(w)


@pytest.mark.parametrize("name", list(WORKLOADS), ids=list(WORKLOADS))
def test_parity_full_workload(name):
    w = WORKLOADS[name]
    _run_and_compare(w)
    torch.cuda.empty_cache()


def test_parity_recompute_cache():
    """Backward without the forward's cache recomputes it; results are bitwise equal."""
    for w in (SMALL[0], SMALL[7]):
        _note(f"[recompute] {w.name}")
        dev = gu.to_dev(workloads.generate(w))
        a = gu.gpu_run(w, dev, use_cache=True)
        b = gu.gpu_run(w, dev, use_cache=False)
        for k in a:
            if a[k] is not None:
                assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("w", [SMALL[0], SMALL[7], SMALL[12]], ids=["hw_bf16", "lr_bf16", "lr_fp32"])
def test_forward_without_cache(w):
    """The forward without a caller cache (generator values in the library's
    workspace slot) gives the same y bitwise, and the backward that then
    recomputes the cache the same gradients."""
    _note(f"[no-cache fwd] {w.name}")
    dev = gu.to_dev(workloads.generate(w))
    a = gu.gpu_run(w, dev)
    b = gu.gpu_run(w, dev, fwd_cache=False, use_cache=False)
    for k in a:
        if a[k] is not None and b.get(k) is not None:
            assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("w", [SMALL[0], SMALL[2], SMALL[7], SMALL[8], SMALL[6], SMALL[12]],
                         ids=["hw_hd72", "hw_hd68", "lr_r16", "lr_r32", "hw_fp32", "lr_fp32"])
def test_optional_outputs(w):
    """dh = NULL (the generator-weight gradient then runs without the dh
    product, on another launch shape) and dw0 = NULL with a bias present: the
    outputs still computed are bitwise those of the full backward, except dW
    / dA, whose token split may differ without dh; those match the oracle."""
    _note(f"[optional outputs] {w.name}")
    inp = workloads.generate(w)
    dev = gu.to_dev(inp)
    full = gu.gpu_run(w, dev)
    ref = gu.oracle_run(w, inp)
    for need_dh, need_dw0 in ((False, True), (True, False), (False, False)):
        part = gu.gpu_run(w, dev, need_dh=need_dh, need_dw0=need_dw0)
        assert ("dh" in part) == need_dh and ("dw0" in part) == (need_dw0 and dev.get("w0") is not None)
        for k in full:
            if full[k] is None or k not in part:
                continue
            if k in ("dW", "dA"):
                gu.compare(w, part, ref, keys=[k])
            else:
                assert torch.equal(full[k], part[k]), (k, need_dh, need_dw0)


def test_deterministic():
    for w in (SMALL[2], SMALL[8]):
        _note(f"[determinism] {w.name}")
        dev = gu.to_dev(workloads.generate(w))
        a = gu.gpu_run(w, dev)
        b = gu.gpu_run(w, dev)
        for k in a:
            if a[k] is not None:
                assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("w", [SMALL[0], SMALL[6], SMALL[7], SMALL[12]],
                         ids=["hw_bf16", "hw_fp32", "lr_bf16", "lr_fp32"])
def test_zero_filter_identity(w):
    """Zero generator and no bias: y == x and dx == dy bitwise."""
    _note(f"[identity] {w.name}")
    w = w.with_(bias_std=0.0)
    inp = workloads.generate(w)
    for key in ("W", "U"):
        if inp.get(key) is not None:
            inp[key] = torch.zeros_like(inp[key])
    dev = gu.to_dev(inp)
    got = gu.gpu_run(w, dev)
    assert torch.equal(got["y"], dev["x"])
    assert torch.equal(got["dx"], dev["dy"])


@pytest.mark.parametrize("w", [SMALL[2], SMALL[7]], ids=["hw", "lr"])
def test_causality(w):
    """Perturbing x and h after token t leaves y up to t bitwise unchanged."""
    _note(f"[causality] {w.name}")
    inp = workloads.generate(w)
    dev = gu.to_dev(inp)
    y0 = gu.gpu_run(w, dev)["y"]
    for t in (0, 1, w.T // 2, w.T - 2):
        d2 = dict(dev)
        x = dev["x"].clone()
        h = dev["h"].clone()
        x[:, t + 1:] += 1.0
        h[:, t + 1:] -= 0.5
        d2["x"], d2["h"] = x, h
        y1 = gu.gpu_run(w, d2)["y"]
        assert torch.equal(y0[:, : t + 1], y1[:, : t + 1]), t
        assert not torch.equal(y0[:, t + 1:], y1[:, t + 1:]), t


@pytest.mark.parametrize("w", [SMALL[0], SMALL[7], _BY_NAME["hw_bf16_hd68_fold_B4"]], ids=["hw", "lr", "hw_fold"])
def test_batch_isolation(w):
    """Changing one sequence's h, x and dy leaves the other sequences' y, dx
    and dh bitwise unchanged (nothing crosses batch rows)."""
    _note(f"[isolation] {w.name}")
    assert w.B >= 2
    dev = gu.to_dev(workloads.generate(w))
    a = gu.gpu_run(w, dev)
    d2 = dict(dev)
    for key, delta in (("x", 1.0), ("h", -0.5), ("dy", 0.25)):
        t = dev[key].clone()
        t[0] += delta
        d2[key] = t
    b = gu.gpu_run(w, d2)
    for key in ("y", "dx", "dh"):
        assert torch.equal(a[key][1:], b[key][1:]), key
        assert not torch.equal(a[key][0], b[key][0]), key


def test_empty_batch():
    """B*T == 0: the forward is a no-op, the backward writes zero weight gradients."""
    w = SMALL[7].with_(B=0)
    inp = workloads.generate(SMALL[7])
    dev = gu.to_dev(inp)
    h = dev["h"][:0]
    x = dev["x"][:0]
    import input_dependent_depthwise_amd as dc
    y = dc.dynconv_fwd(h, x, k=w.k, A=dev["A"], U=dev["U"], w0=dev["w0"])
    assert y.shape == x.shape
    out = {"dA": torch.full((w.d, w.rank), 7.0, device="cuda"),
           "dU": torch.full((w.rank, w.D * w.k), 7.0, device="cuda"),
           "dw0": torch.full((w.D, w.k), 7.0, device="cuda")}
    g = dc.dynconv_bwd(h, x, x, k=w.k, A=dev["A"], U=dev["U"], w0=dev["w0"], out=out)
    torch.cuda.synchronize()
    for k in ("dA", "dU", "dw0"):
        assert torch.count_nonzero(g[k]).item() == 0, k


@pytest.mark.parametrize("w", [SMALL[0], SMALL[7]], ids=["hw", "lr"])
def test_autograd_wrapper(w):
    """DynConvFn gives the direct calls' results bitwise: y, dx, dh, and the
    weight gradients cast to the weights' dtype."""
    _note(f"[autograd] {w.name}")
    dev = gu.to_dev(workloads.generate(w))
    ref = gu.gpu_run(w, dev)
    leaves = {k: (None if dev.get(k) is None else dev[k].clone().requires_grad_(True))
              for k in ("h", "x", "W", "A", "U", "w0")}
    y = dc.DynConvFn.apply(leaves["h"], leaves["x"], leaves["W"], leaves["A"], leaves["U"], leaves["w0"],
                           w.k, w.n_heads)
    y.backward(dev["dy"])
    torch.cuda.synchronize()
    assert torch.equal(y.detach(), ref["y"])
    assert torch.equal(leaves["x"].grad, ref["dx"])
    assert torch.equal(leaves["h"].grad, ref["dh"])
    for key, gkey in (("W", "dW"), ("A", "dA"), ("U", "dU"), ("w0", "dw0")):
        if leaves[key] is not None:
            assert torch.equal(leaves[key].grad, ref[gkey].to(leaves[key].dtype)), key


DECODE = [SMALL[0], SMALL[7], SMALL[6], SMALL[12], SMALL[9], SMALL[5], SMALL[10], SMALL[4],
          SMALL[22], SMALL[25],  # widths that are not whole 16-byte vectors
          # more than 1024 (sequence, 256-channel) blocks: four sequences per block, the
          # last block with one (161 = 4 * 40 + 1)
          Workload("dec_grouped_lr", B=161, T=6, d=64, D=2048, k=4, kind=LOWRANK, rank=16, seed=41),
          Workload("dec_grouped_hw_k3", B=161, T=5, d=64, D=2048, k=3, kind=HEADWISE, n_heads=16, seed=42),
          # the row-wise generator pass: 256 generator columns with 68-channel heads
          # straddling the 256-channel blocks; fp32 rows of 32 and 128 columns; four
          # fp32 sequences per block
          Workload("dec_hw_hd68_N256", B=3, T=40, d=64, D=4352, k=4, kind=HEADWISE, n_heads=64, seed=43),
          Workload("dec_fp32_lr_r32_k3", B=5, T=30, d=48, D=256, k=3, kind=LOWRANK, rank=32, dtype="fp32",
                   seed=44),
          Workload("dec_fp32_hw_N128", B=2, T=30, d=40, D=512, k=4, kind=HEADWISE, n_heads=32, dtype="fp32",
                   seed=45),
          Workload("dec_grouped_fp32_lr", B=161, T=4, d=32, D=2048, k=2, kind=LOWRANK, rank=8, dtype="fp32",
                   seed=46)]


@pytest.mark.parametrize("w", DECODE, ids=[w.name for w in DECODE])
def test_decode_steps_match_forward(w):
    """dynconv_decode, called once per position from a zeroed history, gives
    the oracle's forward rows (first 48 positions of every sequence)."""
    _note(f"[decode] {w.name}")
    inp = workloads.generate(w)
    s = gu.oracle_shape(w)
    ref = oracle.forward(s, inp["h"], inp["x"], W=inp.get("W"), A=inp.get("A"), U=inp.get("U"),
                         w0=inp.get("w0"))["y"]
    dev = gu.to_dev(inp)
    B, T, D = dev["x"].shape
    steps = min(T, 48)
    state = torch.zeros(B, w.k - 1, D, dtype=dev["x"].dtype, device="cuda") if w.k > 1 else None
    kw = dict(k=w.k, W=dev.get("W"), A=dev.get("A"), U=dev.get("U"), w0=dev.get("w0"), n_heads=w.n_heads)
    # (clone: a row of a one-sequence batch is already contiguous, and a view of it
    # would start at an offset that is not 16-byte aligned, which the ABI rejects)
    ys = [dc.dynconv_decode(dev["h"][:, t].clone(), dev["x"][:, t].clone(), state, **kw)
          for t in range(steps)]
    torch.cuda.synchronize()
    y = torch.stack(ys, 1).float().cpu().numpy()
    err = gu.max_rel_err(y, np.asarray(ref).reshape(B, T, D)[:, :steps])
    assert err <= gu.TOL[w.dtype], (w.name, err)
    if w.k > 1:  # the history holds the last k-1 rows of x
        last = dev["x"][:, max(0, steps - (w.k - 1)):steps]
        assert torch.equal(state[:, state.shape[1] - last.shape[1]:], last)


@pytest.mark.parametrize("kind", ["lowrank", "headwise", "headwise_wide"])
def test_near_size_limit_per_sequence(kind):
    """Tensors just under the 2 GiB limit of the fused kernels' 32-bit byte
    offsets.  The oracle cannot run at this size; a property that holds at any
    size stands in: a sequence's y, dx and dh depend only on that sequence
    (tiles are aligned to sequence starts and every reduction has a fixed
    order), so the last sequences of the big batch, where the offsets are
    largest, must equal bitwise a run of those sequences alone.  (The wide
    projection picks its K split by row count, so the tail is large enough,
    32768 rows, to take the same one as the full batch.)"""
    import input_dependent_depthwise_amd as dc
    T, k = 2048, 4
    if kind == "lowrank":
        d, D, rank, n_heads = 768, 2304, 16, 0
    elif kind == "headwise":
        d, D, rank, n_heads = 512, 3072, 0, 24
    else:  # 256 generator columns (projection tile, wide dM) and heads of 68 channels
        d, D, rank, n_heads = 512, 4352, 0, 64
    B = ((1 << 31) - 64 - 1) // (T * D * 2)  # largest batch with B*T*D*2 below the limit
    assert B * T * D * 2 < (1 << 31) - 64
    _note(f"[limit] {kind} B={B} T={T} d={d} D={D} bytes per tensor={B * T * D * 2}")
    gen = torch.Generator(device="cuda").manual_seed(7)
    bf = torch.bfloat16
    h = torch.randn(B, T, d, device="cuda", generator=gen).to(bf)
    x = torch.randn(B, T, D, device="cuda", generator=gen).to(bf)
    dy = torch.randn(B, T, D, device="cuda", generator=gen).to(bf)
    w0 = (0.1 * torch.randn(D, k, device="cuda", generator=gen)).to(bf)
    if kind == "lowrank":
        wk = dict(A=(0.02 * torch.randn(d, rank, device="cuda", generator=gen)).to(bf),
                  U=(0.02 * torch.randn(rank, D * k, device="cuda", generator=gen)).to(bf))
    else:
        wk = dict(W=(0.02 * torch.randn(d, n_heads * k, device="cuda", generator=gen)).to(bf), n_heads=n_heads)

    def run(hh, xx, dd):
        y, cache = dc.dynconv_fwd(hh, xx, k=k, w0=w0, want_cache=True, **wk)
        g = dc.dynconv_bwd(hh, xx, dd, k=k, w0=w0, gen_cache=cache, need_dh=True, need_dw0=True, **wk)
        torch.cuda.synchronize()
        return y, g["dx"], g["dh"]

    tail = 16
    big = run(h, x, dy)
    big = [t[B - tail:].clone() for t in big]
    torch.cuda.empty_cache()
    small = run(h[B - tail:].contiguous(), x[B - tail:].contiguous(), dy[B - tail:].contiguous())
    for name, a, b in zip(("y", "dx", "dh"), big, small):
        assert torch.isfinite(a.float()).all(), name
        assert torch.equal(a, b), f"{kind} {name}: the last sequences differ from a run of them alone"
    del h, x, dy, big, small
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# packed documents: one row holding documents back to back
# ---------------------------------------------------------------------------
def _cu(lens):
    return list(np.cumsum([0] + list(lens)))


# (workload with B = 1 and T = the total, document lengths): documents of 1,
# 2 and 3 tokens (below k), an empty one, and documents spanning several tiles
PACKED_LENS = (1, 2, 3, 70, 0, 5, 130, 33, 64)
PACKED = [
    Workload("pk_hw_bf16_hd68", B=1, T=308, d=96, D=544, k=4, kind=HEADWISE, n_heads=8, seed=71),
    Workload("pk_hw_bf16_hd128_k3", B=1, T=308, d=64, D=1024, k=3, kind=HEADWISE, n_heads=8, seed=72),
    Workload("pk_hw_bf16_hd16_k2", B=1, T=308, d=32, D=256, k=2, kind=HEADWISE, n_heads=16, seed=73),
    Workload("pk_hw_bf16_hd4", B=1, T=308, d=16, D=64, k=4, kind=HEADWISE, n_heads=16, seed=74),
    Workload("pk_hw_bf16_N256", B=1, T=308, d=64, D=512, k=4, kind=HEADWISE, n_heads=64, seed=75),
    Workload("pk_lr_bf16_r16", B=1, T=308, d=128, D=360, k=4, kind=LOWRANK, rank=16, seed=76),
    Workload("pk_lr_bf16_r16_D384", B=1, T=308, d=128, D=384, k=4, kind=LOWRANK, rank=16, seed=83),
    Workload("pk_lr_bf16_r32_k3", B=1, T=308, d=64, D=1024, k=3, kind=LOWRANK, rank=32, seed=77),
    Workload("pk_lr_bf16_r1_k1", B=1, T=308, d=32, D=64, k=1, kind=LOWRANK, rank=1, seed=78),
    Workload("pk_lr_bf16_r64_k8", B=1, T=308, d=64, D=256, k=8, kind=LOWRANK, rank=64, seed=79),
    Workload("pk_hw_fp32_k5", B=1, T=308, d=32, D=48, k=5, kind=HEADWISE, n_heads=3, dtype="fp32", seed=80),
    Workload("pk_lr_fp32", B=1, T=308, d=32, D=64, k=4, kind=LOWRANK, rank=8, dtype="fp32", seed=81),
    Workload("pk_lr_bf16_D100", B=1, T=308, d=64, D=100, k=3, kind=LOWRANK, rank=16, seed=82),
    Workload("pk_hw_bf16_k8", B=1, T=308, d=64, D=512, k=8, kind=HEADWISE, n_heads=8, seed=84),
    Workload("pk_lr_bf16_r16_k8", B=1, T=308, d=128, D=384, k=8, kind=LOWRANK, rank=16, seed=86),
    Workload("pk_lr_bf16_r32_k6", B=1, T=308, d=64, D=256, k=6, kind=LOWRANK, rank=32, seed=87),
    Workload("pk_hw_bf16_k6_hd68", B=1, T=308, d=64, D=544, k=6, kind=HEADWISE, n_heads=8, seed=85),
]


@pytest.mark.parametrize("w", PACKED, ids=[w.name for w in PACKED])
def test_packed_parity(w):
    """Packed documents against the oracle's packed reading (the window stops
    at every document start), element by element."""
    cu = _cu(PACKED_LENS)
    assert cu[-1] == w.T
    _note(f"[packed] {w.name} D={w.D} k={w.k} {w.kind} {w.dtype} docs={PACKED_LENS}")
    inp = workloads.generate(w)
    got = gu.gpu_run(w, gu.to_dev(inp), cu_seqlens=cu)
    ref = gu.oracle_run(w, inp, cu_seqlens=cu)
    errs = gu.compare(w, got, ref)
    _note(f"[packed] {w.name} errors {errs}")


@pytest.mark.parametrize("name", ["mamba2_inconv_headwise", "qkv_150m_lowrank"])
def test_packed_equal_documents_are_the_batch(name):
    """At full size: the B sequences of a workload packed into one row as B
    documents give the batched run's outputs bitwise (the launch layouts
    depend on the token count only, and the document table reproduces the
    batch's sequence starts)."""
    w = WORKLOADS[name]
    _note(f"[packed full] {name}")
    dev = gu.to_dev(workloads.generate(w))
    a = gu.gpu_run(w, dev)
    wp = w.with_(B=1, T=w.B * w.T)
    devp = {k: (None if v is None else (v.reshape(1, w.B * w.T, -1) if k in ("h", "x", "dy") else v))
            for k, v in dev.items()}
    b = gu.gpu_run(wp, devp, cu_seqlens=[i * w.T for i in range(w.B + 1)])
    for k in a:
        if a[k] is not None:
            assert torch.equal(a[k].reshape(-1), b[k].reshape(-1)), k
    del dev, devp, a, b
    torch.cuda.empty_cache()


def test_packed_autograd_wrapper():
    """DynConvFn with cu_seqlens equals the direct packed calls bitwise."""
    w = PACKED[0]
    cu = torch.tensor(_cu(PACKED_LENS), dtype=torch.int32, device="cuda")
    dev = gu.to_dev(workloads.generate(w))
    ref = gu.gpu_run(w, dev, cu_seqlens=_cu(PACKED_LENS))
    leaves = {k: (None if dev.get(k) is None else dev[k].clone().requires_grad_(True))
              for k in ("h", "x", "W", "w0")}
    y = dc.DynConvFn.apply(leaves["h"], leaves["x"], leaves["W"], None, None, leaves["w0"], w.k, w.n_heads, cu)
    y.backward(dev["dy"])
    torch.cuda.synchronize()
    assert torch.equal(y.detach(), ref["y"])
    assert torch.equal(leaves["x"].grad, ref["dx"])
    assert torch.equal(leaves["h"].grad, ref["dh"])


@pytest.mark.parametrize("kind", ["headwise", "lowrank"])
def test_large_batch_runs_in_chunks(kind):
    """Batches whose tensors pass the tuned kernels' 2 GiB offset limit run as
    chunks of whole sequences on those kernels (the largest chunk that fits,
    then the rest).  Every per-sequence output equals, bitwise, a run of that
    chunk alone, and each weight gradient is the first chunk's plus the
    second's (one fp32 addition, in chunk order)."""
    import input_dependent_depthwise_amd as dc
    k = 4
    if kind == "headwise":  # Mamba-2 channels: 15 sequences per chunk
        T, d, D, B, first = 16384, 512, 4352, 16, 15
        gen_cols = 64 * k
    else:  # 150M QKV channels: 227 sequences per chunk
        T, d, D, B, first = 2048, 768, 2304, 230, 227
        gen_cols = 16
    assert first * T * D * 2 < (1 << 31) - 64 <= (first + 1) * T * D * 2 and B > first
    _note(f"[chunks] {kind} B={B} T={T} d={d} D={D} bytes per tensor={B * T * D * 2}")
    gen = torch.Generator(device="cuda").manual_seed(11)
    bf = torch.bfloat16
    h = torch.randn(B, T, d, device="cuda", generator=gen).to(bf)
    x = torch.randn(B, T, D, device="cuda", generator=gen).to(bf)
    dy = torch.randn(B, T, D, device="cuda", generator=gen).to(bf)
    w0 = (0.1 * torch.randn(D, k, device="cuda", generator=gen)).to(bf)
    if kind == "headwise":
        wk = dict(W=(0.02 * torch.randn(d, gen_cols, device="cuda", generator=gen)).to(bf), n_heads=64)
        grads = ("dW", "dw0")
    else:
        wk = dict(A=(0.02 * torch.randn(d, gen_cols, device="cuda", generator=gen)).to(bf),
                  U=(0.02 * torch.randn(gen_cols, D * k, device="cuda", generator=gen)).to(bf))
        grads = ("dA", "dU", "dw0")

    def run(hh, xx, dd):
        y, cache = dc.dynconv_fwd(hh, xx, k=k, w0=w0, want_cache=True, **wk)
        g = dc.dynconv_bwd(hh, xx, dd, k=k, w0=w0, gen_cache=cache, need_dh=True, need_dw0=True, **wk)
        torch.cuda.synchronize()
        return {"y": y, "cache": cache.view(hh.shape[0], T, -1), **g}

    full = run(h, x, dy)
    parts = [run(h[a:b].contiguous(), x[a:b].contiguous(), dy[a:b].contiguous()) for a, b in ((0, first), (first, B))]
    for key in ("y", "cache", "dx", "dh"):
        assert torch.isfinite(full[key].float()).all(), key
        assert torch.equal(full[key][:first], parts[0][key]), (kind, key, "first chunk")
        assert torch.equal(full[key][first:], parts[1][key]), (kind, key, "second chunk")
    for key in grads:
        assert torch.equal(full[key], parts[0][key] + parts[1][key]), (kind, key)
    del h, x, dy, full, parts
    torch.cuda.empty_cache()
