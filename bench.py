#!/usr/bin/env python3
"""Benchmark of the dynamic short convolution layer, forward + backward, on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch: dynconv_fwd
(generator projection u = hW or z = hA, filter formation, causal depthwise
conv + residual) then dynconv_bwd (dx, dh, dW or dA and dU, dw0), both
through the C ABI, on synthetic seeded inputs already resident in HBM.
Inputs, outputs and workspaces are preallocated; several copies of the
input set rotate from step to step so that the 256 MB Infinity Cache cannot
hold one step's working set for the next.

Prints one JSON line: tokens/s of the whole job (``value``), the roofline of
the dominant kernel (its average launch time measured live with HIP events
recorded on the library's stream around that kernel on every fourth timed
step, algorithmic bytes per launch / that time, against 8 TB/s), and the fp64
CPU oracle timed on the host cores on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 matrix-core peak, published
MALL_BYTES = 256 * 2**20     # Infinity Cache
MAX_SETS = 8                 # rotating input sets at most (small workloads fit in the cache anyway)
PROFILES = os.path.join(ROOT, "profiles")


def algorithmic_bytes(w: workloads.Workload) -> dict:
    """Bytes per token the layer must move (inputs read once, outputs written once).

    forward : h (d) + x (D) read, y (D) written                       -> eb*(d + 2D)
    backward: h, x, dy read; dx, dh written                           -> eb*(2d + 3D)
    fused bwd conv kernel: x, dy read, dx written                     -> eb*3D
    fused fwd conv kernel: x read, y written                          -> eb*2D
    """
    eb, d, D = w.elem_bytes, w.d, w.D
    return {"fwd": eb * (d + 2 * D), "bwd": eb * (2 * d + 3 * D), "step": eb * (3 * d + 5 * D),
            "bwd_conv": eb * 3 * D, "fwd_conv": eb * 2 * D}


def generator_flops(w: workloads.Workload) -> dict:
    """Matrix-core flops per launch of the generator kernels (dense bf16 GEMMs).

    gen_proj: u = h W or z = h A                        -> 2 * BT * d * N
    gen_bwd : dh = g M^T and dM = h^T g (M = W or A)     -> 4 * BT * d * N
    """
    n = w.gen_cols
    return {"gen_proj": 2 * w.tokens * w.d * n, "gen_bwd": 4 * w.tokens * w.d * n}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# Sources each roofline kernel is built from (its own file, the headers it
# includes, the public header): a traffic record counts only while these are
# unchanged.
KERNEL_SOURCES = {
    ("bwd_conv", "headwise"): ["conv_bwd_headwise.hip"],
    ("bwd_conv", "lowrank"): ["conv_bwd_lowrank.hip", "mfma.h"],
    ("fwd_conv", "headwise"): ["conv_fwd_headwise.hip"],
    ("fwd_conv", "lowrank"): ["conv_fwd_lowrank.hip", "mfma.h"],
}
COMMON_SOURCES = ["bufio.h", "common.h", "kernels.h", "../../include/dynconv.h"]
# the symbol of each roofline kernel in a rocprofv3 trace (substring)
KERNEL_SYMBOLS = {("bwd_conv", "headwise"): "k_bwd_hw", ("bwd_conv", "lowrank"): "k_bwd_lr",
                  ("fwd_conv", "headwise"): "k_fwd_h", ("fwd_conv", "lowrank"): "k_fwd_lowrank"}


def kernel_source_sha(kernel: str, kind: str) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "input_dependent_depthwise_amd", "csrc")
    for f in KERNEL_SOURCES[(kernel, kind)] + COMMON_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(os.path.basename(f).encode() + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, w: workloads.Workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken from the kernel's current sources; else None."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{w.name}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha") != kernel_source_sha(kernel, w.kind):
        return None
    return rec.get("bytes_per_launch")


def _counter_per_dispatch(path: str, counter: str) -> dict:
    """Mean value of one counter per kernel name from a rocprofv3 counter CSV."""
    import csv
    tot, cnt = {}, {}
    for r in csv.DictReader(open(path)):
        if r.get("Counter_Name") != counter:
            continue
        k = r["Kernel_Name"]
        tot[k] = tot.get(k, 0.0) + float(r["Counter_Value"])
        cnt[k] = cnt.get(k, 0) + 1
    return {k: tot[k] / cnt[k] for k in tot}


def traffic_record(args, paths) -> int:
    """Writes the traffic record of the roofline kernel (and prints a table of
    every kernel) from four rocprofv3 --pmc CSVs: FETCH_SIZE and WRITE_SIZE of
    the workload, then of --copy-calibration 512.  Each counter is scaled by
    what it reads for the plain copy of known size."""
    w = workloads.WORKLOADS[args.workload]
    fetch, write, cf, cw = (_counter_per_dispatch(p, c) for p, c in
                            zip(paths, ("FETCH_SIZE", "WRITE_SIZE", "FETCH_SIZE", "WRITE_SIZE")))
    copy_kib = 512 * 1024
    f_scale = copy_kib / max(cf.values())   # the copy reads 512 MiB
    w_scale = copy_kib / max(cw.values())   # and writes 512 MiB
    sym = KERNEL_SYMBOLS[(args.roofline_kernel, w.kind)]
    rows = []
    for k in sorted(fetch, key=lambda k: -fetch[k] - write.get(k, 0.0)):
        rd, wr = fetch[k] * f_scale * 1024, write.get(k, 0.0) * w_scale * 1024
        rows.append((k, fetch[k], write.get(k, 0.0), rd / 1e6, wr / 1e6))
    dom = [r for r in rows if sym in r[0]]
    if not dom:
        print(f"bench.py --traffic-record: no kernel matching {sym}", file=sys.stderr)
        return 2
    k, fk, wk, rd, wr = dom[0]
    alg = algorithmic_bytes(w)[args.roofline_kernel] * w.tokens
    rec = {"kernel": args.roofline_kernel, "kernel_symbol": k, "workload": w.name,
           "source_sha": kernel_source_sha(args.roofline_kernel, w.kind),
           "source_files": KERNEL_SOURCES[(args.roofline_kernel, w.kind)] + COMMON_SOURCES,
           "bytes_per_launch": int(round((rd + wr) * 1e6)), "fetch_kib_per_dispatch": round(fk, 1),
           "write_kib_per_dispatch": round(wk, 1), "fetch_scale": round(f_scale, 4),
           "write_scale": round(w_scale, 4), "algorithmic_bytes_per_launch": alg}
    out = args.traffic_out or os.path.join(PROFILES, f"traffic_{args.roofline_kernel}_{w.name}.json")
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    print(f"| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled MB read | scaled MB written |")
    print(f"|---|---|---|---|---|")
    for k, fk, wk, rd, wr in rows:
        print(f"| `{k}` | {fk:.0f} | {wk:.0f} | {rd:.1f} | {wr:.1f} |")
    print(f"\nscales: FETCH_SIZE {f_scale:.4f}, WRITE_SIZE {w_scale:.4f}; record written to {out}")
    return 0


def cpu_baseline(w: workloads.Workload, inp: dict, budget_s: float) -> dict:
    """fp64 oracle (plain C loops, OpenMP) on a bounded sample of the workload."""
    import oracle  # test infrastructure: only this leg of the benchmark uses it

    # sample: the first n sequences, n chosen from a one-sequence probe so the
    # timed run stays within the budget
    def run(nseq):
        s = oracle.Shape(B=nseq, T=w.T, d=w.d, D=w.D, k=w.k,
                         kind=oracle.HEADWISE if w.kind == workloads.HEADWISE else oracle.LOWRANK,
                         n_heads=w.n_heads, rank=w.rank)
        args = {k: inp.get(k) for k in ("W", "A", "U", "w0")}
        t0 = time.perf_counter()
        fw = oracle.forward(s, inp["h"][:nseq], inp["x"][:nseq], **args)
        oracle.backward(s, inp["h"][:nseq], inp["x"][:nseq], inp["dy"][:nseq], w=fw["w"], **args)
        return time.perf_counter() - t0

    t1 = run(1)
    nseq = max(1, min(w.B, int(budget_s / max(t1, 1e-6))))
    t = run(nseq) if nseq > 1 else t1
    # a whole workload that takes well under the budget is run again, so that the
    # rate comes from about budget_s of work
    reps = 1
    if nseq == w.B and t < budget_s / 2:
        extra = min(30, int(budget_s / max(t, 1e-6)) - 1)
        t += sum(run(nseq) for _ in range(extra))
        reps += extra
    tokens = nseq * w.T * reps
    return {"value": round(tokens / t, 1), "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle", "affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
            "sample": f"{nseq} of {w.B} sequences of {w.name}, fwd+bwd, fp64, {reps} run(s), "
                      f"{tokens} tokens in {t:.2f} s on {oracle.num_threads()} OpenMP threads"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=workloads.BENCH_WORKLOAD, choices=list(workloads.WORKLOADS))
    ap.add_argument("--sets", type=int, default=0,
                    help=f"rotating input sets (0: enough to exceed 2x MALL, at most {MAX_SETS})")
    ap.add_argument("--mfma-steps", type=int, default=8,
                    help="after the timed steps, this many more steps time the generator kernels "
                         "with HIP events (matrix-core roofline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--trace-every", type=int, default=4,
                    help="time the dominant kernel with HIP events on every N-th timed step")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    ap.add_argument("--roofline-kernel", default="bwd_conv", choices=["bwd_conv", "fwd_conv"],
                    help="kernel whose roofline is reported (the dominant one by default)")
    ap.add_argument("--decode", type=int, default=0, metavar="B",
                    help="instead of the training step, time dynconv_decode (one new token for each "
                         "of B sequences) on the workload's layer shape")
    ap.add_argument("--proj", action="store_true",
                    help="instead of the training step, time the forward with the producing "
                         "projection fused in (dynconv_fwd_proj) beside torch.matmul + dynconv_fwd")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the layer, run --steps device copies of MIB MiB (a plain copy "
                         "kernel of known size, to scale the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--traffic-record", nargs=4, metavar="CSV",
                    help="no GPU: build the roofline kernel's traffic record from four rocprofv3 "
                         "--pmc counter CSVs (FETCH_SIZE, WRITE_SIZE of the workload, then of "
                         "--copy-calibration 512)")
    ap.add_argument("--traffic-out", default="", help="where --traffic-record writes (default: profiles/)")
    args = ap.parse_args()

    if args.traffic_record:
        return traffic_record(args, args.traffic_record)

    if args.copy_calibration:
        import torch
        n = args.copy_calibration * 2**20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / args.steps
        print(json.dumps({"copy_bytes": n, "steps": args.steps, "ms_per_copy": round(dt * 1e3, 4),
                          "gbs": round(2 * n / dt / 1e9, 1)}), flush=True)
        return 0

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the layer shards over batch, sequence or channels, but no multi-GPU path is "
              "built here)", file=sys.stderr)
        return 2

    import torch
    import input_dependent_depthwise_amd as dc

    if args.decode:
        return bench_decode(args, torch, dc)
    if args.proj:
        return bench_proj(args, torch, dc)

    w = workloads.WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    inp = workloads.generate(w)

    # --- device buffers: R rotating sets ---
    per_set = (w.tokens * (2 * w.d + 4 * w.D) * w.elem_bytes)  # h, x, dy, y, dx, dh
    R = args.sets or min(MAX_SETS, max(2, -(-2 * MALL_BYTES // per_set) + 1))
    prob = dc.make_problem(inp["x"], inp["h"], w.k)
    sets = []
    for _ in range(R):
        s = {k: (None if v is None else v.to(dev)) for k, v in inp.items()}
        gen = dc.make_gen(s.get("W"), s.get("A"), s.get("U"), s.get("w0"), w.n_heads)
        s["gen"] = gen
        s["y"] = torch.empty_like(s["x"])
        s["cache"] = torch.empty(w.tokens, w.gen_cols, dtype=torch.float32, device=dev)
        s["ws_f"] = torch.empty(max(1, dc.dynconv_workspace_bytes(prob, gen, 0)), dtype=torch.uint8, device=dev)
        s["ws_b"] = torch.empty(max(1, dc.dynconv_workspace_bytes(prob, gen, 1)), dtype=torch.uint8, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        s["out"] = {"dx": torch.empty_like(s["x"]), "dh": torch.empty_like(s["h"]),
                    "dw0": torch.empty(w.D, w.k, **f32)}
        if w.kind == workloads.HEADWISE:
            s["out"]["dW"] = torch.empty(w.d, w.gen_cols, **f32)
        else:
            s["out"]["dA"] = torch.empty(w.d, w.rank, **f32)
            s["out"]["dU"] = torch.empty(w.rank, w.D * w.k, **f32)
        sets.append(s)
    kw = dict(k=w.k, n_heads=w.n_heads)

    def step(i, trace=None):
        s = sets[i % R]
        g = dict(W=s.get("W"), A=s.get("A"), U=s.get("U"), w0=s.get("w0"))
        if trace is not None and trace[0] == "fwd":
            dc.dynconv_trace_next(trace[1], trace[2], trace[3])
        dc.dynconv_fwd(s["h"], s["x"], y=s["y"], gen_cache=s["cache"], workspace=s["ws_f"], **g, **kw)
        if trace is not None and trace[0] == "bwd":
            dc.dynconv_trace_next(trace[1], trace[2], trace[3])
        dc.dynconv_bwd(s["h"], s["x"], s["dy"], gen_cache=s["cache"], out=s["out"], workspace=s["ws_b"],
                       **g, **kw)

    # dominant kernel: the fused backward conv (largest algorithmic traffic)
    dom = {"bwd_conv": ("bwd", dc.DYNCONV_K_BWD_CONV, "bwd_conv"),
           "fwd_conv": ("fwd", dc.DYNCONV_K_FWD_CONV, "fwd_conv")}[args.roofline_kernel]
    # every trace_every-th timed step carries the kernel's events: an event
    # between two kernels holds the second one back until the first has
    # finished and the event is processed (a few µs of idle GPU each), which
    # the untraced steps do not pay
    traced = list(range(0, args.steps, max(1, args.trace_every)))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in traced]
    for a, b in ev:  # create the underlying HIP events
        a.record()
        b.record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    print(f"[bench] {w.name}: warmup {args.warmup} done, {R} rotating sets, timing {args.steps} steps",
          file=sys.stderr, flush=True)

    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    tr = {t: e for t, e in zip(traced, ev)}
    for i in range(args.steps):
        e = tr.get(i)
        step(args.warmup + i, trace=None if e is None else (dom[0], dom[1], e[0], e[1]))
    t_stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t_start.elapsed_time(t_stop) / args.steps
    kern_ms = sum(a.elapsed_time(b) for a, b in ev) / len(ev)

    # matrix-core roofline of the generator kernels, from extra (untimed) steps
    # so that their events do not stretch the timed ones
    mfma = None
    if args.mfma_steps > 0 and w.dtype == "bf16":
        fl = generator_flops(w)
        mev = {k: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.mfma_steps)] for k in ("gen_proj", "gen_bwd")}
        for evs in mev.values():  # create the underlying HIP events
            for a, b in evs:
                a.record()
                b.record()
        for i in range(args.mfma_steps):
            s_ = sets[i % R]
            g = dict(W=s_.get("W"), A=s_.get("A"), U=s_.get("U"), w0=s_.get("w0"))
            a, b = mev["gen_proj"][i]
            dc.dynconv_trace_next(dc.DYNCONV_K_GEN_PROJ, a, b)
            dc.dynconv_fwd(s_["h"], s_["x"], y=s_["y"], gen_cache=s_["cache"], workspace=s_["ws_f"], **g, **kw)
            a, b = mev["gen_bwd"][i]
            dc.dynconv_trace_next(dc.DYNCONV_K_GEN_BWD, a, b)
            dc.dynconv_bwd(s_["h"], s_["x"], s_["dy"], gen_cache=s_["cache"], out=s_["out"],
                           workspace=s_["ws_b"], **g, **kw)
        torch.cuda.synchronize()
        mfma = {"bound": "mfma", "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s", "dtype": "bf16"}
        for k, evs in mev.items():
            kms = sum(a.elapsed_time(b) for a, b in evs) / len(evs)
            tf = fl[k] / (kms / 1e3) / 1e12
            mfma[k] = {"achieved": round(tf, 1), "frac": round(tf / MFMA_BF16_PEAK_TFS, 4),
                       "flops_per_launch": fl[k], "kernel_ms": round(kms, 5)}

    ab = algorithmic_bytes(w)
    value = w.tokens / (ms / 1e3)
    dom_bytes = ab[dom[2]] * w.tokens
    achieved = dom_bytes / (kern_ms / 1e3) / 1e9
    traffic = measured_traffic(dom[2], w)
    line = {
        "metric": "dynconv fwd+bwd tokens/s", "value": round(value, 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) generator, N(0,0.1) bias)",
        "config": {**w.describe(), "tokens_per_step": w.tokens, "rotating_sets": R},
        "step_hbm_gbs": round(ab["step"] * w.tokens / (ms / 1e3) / 1e9, 1),
        "roofline": {"bound": "hbm", "kernel": dom[2], "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel_ms": round(kern_ms, 5),
                     "algorithmic_bytes_per_launch": dom_bytes, "traced_launches": len(ev)},
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
    }
    if mfma is not None:
        line["mfma_roofline"] = mfma
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_budget)
    print(json.dumps(line), flush=True)
    return 0


def bench_decode(args, torch, dc) -> int:
    """Decode steps: B sequences, one token each per step, on the workload's
    layer shape (d_model, D, k, generator).  Inputs are synthetic (seeded
    normal h and x, the workload's generator and bias distributions); 16
    different token rows rotate, and the history is updated in place."""
    w = workloads.WORKLOADS[args.workload]
    B = args.decode
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    g = torch.Generator().manual_seed(100 + w.seed)
    rows = 16
    h = (torch.randn(rows, B, w.d, generator=g)).to(dt).cuda()
    x = (torch.randn(rows, B, w.D, generator=g)).to(dt).cuda()
    wts = {}
    if w.kind == workloads.HEADWISE:
        wts["W"] = (torch.randn(w.d, w.n_heads * w.k, generator=g) * w.gen_std).to(dt).cuda()
    else:
        wts["A"] = (torch.randn(w.d, w.rank, generator=g) * w.gen_std).to(dt).cuda()
        wts["U"] = (torch.randn(w.rank, w.D * w.k, generator=g) * w.gen_std).to(dt).cuda()
    wts["w0"] = (torch.randn(w.D, w.k, generator=g) * w.bias_std).to(dt).cuda() if w.bias_std > 0 else None
    state = torch.zeros(B, w.k - 1, w.D, dtype=dt, device="cuda") if w.k > 1 else None
    y = torch.empty(B, w.D, dtype=dt, device="cuda")
    kw = dict(k=w.k, n_heads=w.n_heads, y=y, **wts)

    def step(i):
        dc.dynconv_decode(h[i % rows], x[i % rows], state, **kw)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(args.steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / args.steps
    eb = 2 if dt == torch.bfloat16 else 4
    wbytes = sum(t.numel() for t in wts.values() if t is not None) * eb
    per_seq = (w.d + 2 * w.D + 2 * (w.k - 1) * w.D) * eb  # h, x, y, history read and written
    nbytes = wbytes + B * per_seq
    line = {"metric": "dynconv decode tokens/s", "value": round(B / (us / 1e6), 1), "unit": "tokens/s",
            "us_per_step": round(us, 3), "batch": B, "steps": args.steps, "warmup": args.warmup,
            "dtype": w.dtype, "data": "synthetic (seeded normal h, x; workload's generator and bias scales)",
            "config": {"workload": w.name, "d_model": w.d, "D": w.D, "k": w.k, "generator": w.describe()["generator"]},
            "roofline": {"bound": "hbm", "achieved": round(nbytes / (us / 1e6) / 1e9, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(nbytes / (us / 1e6) / 1e9 / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes_per_step": nbytes}}
    print(json.dumps(line), flush=True)
    return 0


def bench_proj(args, torch, dc) -> int:
    """The forward with its producing projection: x = h Wp, then the layer on
    x, as one dynconv_fwd_proj call (one matrix-core pass over h writes x and
    the generator values) against torch.matmul(h, Wp) followed by dynconv_fwd
    (two passes over h).  Inputs: the workload's seeded h and generator, Wp
    from workloads.generate_proj_weight; two rotating sets."""
    w = workloads.WORKLOADS[args.workload]
    if w.dtype != "bf16":
        print("bench.py --proj: the fused projection is timed on bf16 workloads", file=sys.stderr)
        return 2
    inp = workloads.generate(w, with_dy=False)
    Wp = workloads.generate_proj_weight(w).cuda()
    R = 2
    sets = []
    for _ in range(R):
        s = {k: (None if v is None else v.cuda()) for k, v in inp.items() if k != "x"}
        s["x"] = torch.empty(w.B, w.T, w.D, dtype=torch.bfloat16, device="cuda")
        s["y"] = torch.empty_like(s["x"])
        s["cache"] = torch.empty(w.tokens, w.gen_cols, dtype=torch.float32, device="cuda")
        sets.append(s)
    prob = dc.make_problem(sets[0]["x"], sets[0]["h"], w.k)
    gen = dc.make_gen(sets[0].get("W"), sets[0].get("A"), sets[0].get("U"), sets[0].get("w0"), w.n_heads)
    ws = torch.empty(max(1, dc.dynconv_workspace_bytes(prob, gen, dc.DYNCONV_WS_CACHED)), dtype=torch.uint8,
                     device="cuda")

    def g(s):
        return dict(W=s.get("W"), A=s.get("A"), U=s.get("U"), w0=s.get("w0"), k=w.k, n_heads=w.n_heads)

    def fused(i, trace=None):
        s = sets[i % R]
        if trace is not None:
            dc.dynconv_trace_next(dc.DYNCONV_K_GEN_PROJ, trace[0], trace[1])
        dc.dynconv_fwd_proj(s["h"], Wp, x=s["x"], y=s["y"], gen_cache=s["cache"], workspace=ws, **g(s))

    def separate(i, trace=None):
        s = sets[i % R]
        torch.matmul(s["h"], Wp, out=s["x"])
        dc.dynconv_fwd(s["h"], s["x"], y=s["y"], gen_cache=s["cache"], workspace=ws, **g(s))

    def timed(fn, n_ev=0):
        for i in range(args.warmup):
            fn(i)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_ev)]
        for a, b in ev:
            a.record()
            b.record()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for i in range(args.steps):
            fn(args.warmup + i)
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / args.steps
        for i, e in enumerate(ev):  # untimed steps: the fused GEMM's own duration
            fn(i, trace=e)
        torch.cuda.synchronize()
        kms = sum(a.elapsed_time(b) for a, b in ev) / len(ev) if ev else None
        return ms, kms

    ms_f, kms = timed(fused, n_ev=max(1, args.mfma_steps))
    print(f"[bench] {w.name}: fused {ms_f:.4f} ms/step", file=sys.stderr, flush=True)
    ms_s, _ = timed(separate)
    flops = 2 * w.tokens * w.d * (w.D + w.gen_cols)
    tf = flops / (kms / 1e3) / 1e12
    line = {"metric": "dynconv fwd with producing projection tokens/s", "value": round(w.tokens / (ms_f / 1e3), 1),
            "unit": "tokens/s", "ms_per_step": round(ms_f, 4), "steps": args.steps, "warmup": args.warmup,
            "higher_is_better": True, "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) h, N(0,1/d_model) Wp, the workload's generator and bias)",
            "config": {**w.describe(), "tokens_per_step": w.tokens},
            "separate": {"what": "torch.matmul(h, Wp) then dynconv_fwd", "ms_per_step": round(ms_s, 4),
                         "tokens_per_s": round(w.tokens / (ms_s / 1e3), 1)},
            "speedup_vs_separate": round(ms_s / ms_f, 3),
            "roofline": {"bound": "mfma", "kernel": "proj_fused", "achieved": round(tf, 1),
                         "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFS, 4),
                         "flops_per_launch": flops, "kernel_ms": round(kms, 5)}}
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
