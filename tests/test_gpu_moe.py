"""MoE per-expert shapes on the GPU against the fp64 oracle.

Inside an expert the layer sees only the tokens routed to it.  The reading
taken here: for each sequence, that expert's tokens keep their order and form
one document of the expert's packed row, so the causal window never crosses
from one sequence to the next (cu_seqlens = per-sequence routed counts, some
of them zero).  Each expert has its own generator weights, so each is one
call.  Expert widths are small (256 or 512 channels) and token counts ragged
(skewed top-1 routing of 4 sequences of 256 tokens over 8 experts).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import workloads
from tests import gpu_util as gu
from workloads import HEADWISE, LOWRANK, Workload

pytestmark = pytest.mark.gpu

N_SEQS, T_SEQ, N_EXPERTS = 4, 256, 8

EXPERTS = {
    "lr_r8_k3": Workload("moe_lr", B=1, T=1, d=512, D=256, k=3, kind=LOWRANK, rank=8, seed=300),
    "hw_h4_k4": Workload("moe_hw", B=1, T=1, d=512, D=512, k=4, kind=HEADWISE, n_heads=4, seed=400),
    "hw_h8_k2_fp32": Workload("moe_hw32", B=1, T=1, d=256, D=256, k=2, kind=HEADWISE, n_heads=8, dtype="fp32",
                              seed=500),
}


@pytest.mark.parametrize("name", list(EXPERTS))
def test_moe_experts(name):
    base = EXPERTS[name]
    counts = workloads.moe_routing(N_SEQS, T_SEQ, N_EXPERTS, seed=base.seed)
    for e in range(N_EXPERTS):
        per_seq = [counts[b][e] for b in range(N_SEQS)]
        cu = [int(c) for c in np.cumsum([0] + per_seq)]
        w = base.with_(name=f"{base.name}_e{e}", T=cu[-1], seed=base.seed + e + 1)
        print(f"[moe] {name} expert {e}: tokens per sequence {per_seq}", flush=True)
        sys.stdout.flush()
        inp = workloads.generate(w)
        got = gu.gpu_run(w, gu.to_dev(inp), cu_seqlens=cu)
        ref = gu.oracle_run(w, inp, cu_seqlens=cu)
        errs = gu.compare(w, got, ref)
        print(f"[moe] {name} expert {e}: errors {errs}", flush=True)
