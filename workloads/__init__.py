"""Seeded synthetic workloads for the dynamic short convolution layer.

This module only draws random inputs; it holds none of the layer's
arithmetic, so both the oracle side (tests) and the GPU side (tests, bench)
take their inputs from here.

Five workloads, named by what they model:

* ``tiny_fp32_headwise``  B=1 T=256 d_model=64 D=64 k=4, head-wise, 4 heads of
  16 channels, fp32.  Small enough for the oracle to finish instantly.
* ``qkv_150m_lowrank``    B=8 T=2048 d_model=768, x = concat(Q,K,V) with
  D=2304, k=4, low-rank rank 16 + static bias, bf16 I/O.
* ``qkv_2b_gqa_headwise`` B=4 T=4096 d_model=2048, Q 2048 + K 512 + V 512
  channels (D=3072), k=4, head-wise over 24 consecutive groups of 128
  channels (16 query heads, 4 key heads, 4 value heads), bf16.
* ``mlp_up_lowrank``      B=4 T=4096 d_model=2048, MLP up-projection output
  D=8192, k=3, low-rank rank 32 + bias, bf16; x drawn as SiLU(a)*b with a, b
  i.i.d. N(0,1) to mimic gated MLP activations.
* ``mamba2_inconv_headwise`` B=2 T=16384 d_model=2048, D=4096+2*128=4352
  (x, B, C streams), k=4, head-wise over 64 consecutive groups of 68
  channels, bf16.

Every tensor is drawn on the host with ``torch.Generator().manual_seed(seed)``
as fp32 ``randn``, scaled, then cast to the I/O dtype, in the fixed order
h, x, generator (W, or A then U), w0, dy.  The oracle widens exactly these
stored values to fp64, so both sides see identical bits.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import torch

HEADWISE = "headwise"
LOWRANK = "lowrank"


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    d: int            # d_model, width of the hidden state h
    D: int            # channels of the convolved sequence x
    k: int            # filter width (taps)
    kind: str         # HEADWISE or LOWRANK
    n_heads: int = 0
    rank: int = 0
    dtype: str = "bf16"   # I/O dtype: "fp32" or "bf16"
    seed: int = 0
    gen_std: float = 0.02   # std of W (head-wise) or A and U (low-rank)
    bias_std: float = 0.1   # std of the static bias w0; 0 disables it
    x_dist: str = "normal"  # "normal" or "silu_gated"

    @property
    def tokens(self) -> int:
        return self.B * self.T

    @property
    def gen_cols(self) -> int:
        return self.n_heads * self.k if self.kind == HEADWISE else self.rank

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "fp32" else 2

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    def describe(self) -> dict:
        g = (f"head-wise {self.n_heads}x{self.D // self.n_heads}" if self.kind == HEADWISE
             else f"low-rank r={self.rank}")
        return {"workload": self.name, "B": self.B, "T": self.T, "d_model": self.d, "D": self.D,
                "k": self.k, "generator": g, "bias": self.bias_std > 0, "io_dtype": self.dtype}


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_fp32_headwise", B=1, T=256, d=64, D=64, k=4, kind=HEADWISE, n_heads=4,
                 dtype="fp32", seed=0),
        Workload("qkv_150m_lowrank", B=8, T=2048, d=768, D=2304, k=4, kind=LOWRANK, rank=16,
                 seed=1),
        Workload("qkv_2b_gqa_headwise", B=4, T=4096, d=2048, D=3072, k=4, kind=HEADWISE,
                 n_heads=24, seed=2),
        Workload("mlp_up_lowrank", B=4, T=4096, d=2048, D=8192, k=3, kind=LOWRANK, rank=32,
                 seed=3, x_dist="silu_gated"),
        Workload("mamba2_inconv_headwise", B=2, T=16384, d=2048, D=4352, k=4, kind=HEADWISE,
                 n_heads=64, seed=4),
    ]
}

# The workload the benchmark times by default: the largest one that fits one
# GPU, the Mamba-2 input convolution (B=2, T=16384, D=4352, 1.83 GB of
# algorithmic traffic per fwd+bwd step).  The others run with --workload.
BENCH_WORKLOAD = "mamba2_inconv_headwise"


def generate(w: Workload, with_dy: bool = True) -> dict:
    """Draw the seeded inputs of ``w`` on the host.

    Returns a dict of CPU tensors in the I/O dtype: h[B,T,d], x[B,T,D],
    W[d, n_heads*k] or A[d,r] and U[r, D*k], w0[D,k] (None when bias_std is 0)
    and dy[B,T,D].
    """
    g = torch.Generator().manual_seed(w.seed)
    dt = w.torch_dtype

    def randn(*shape, std=1.0):
        return (torch.randn(*shape, generator=g, dtype=torch.float32) * std).to(dt)

    out = {"h": randn(w.B, w.T, w.d)}
    if w.x_dist == "silu_gated":
        a = torch.randn(w.B, w.T, w.D, generator=g, dtype=torch.float32)
        b = torch.randn(w.B, w.T, w.D, generator=g, dtype=torch.float32)
        out["x"] = (torch.nn.functional.silu(a) * b).to(dt)
        del a, b
    else:
        out["x"] = randn(w.B, w.T, w.D)
    if w.kind == HEADWISE:
        out["W"] = randn(w.d, w.n_heads * w.k, std=w.gen_std)
    else:
        out["A"] = randn(w.d, w.rank, std=w.gen_std)
        out["U"] = randn(w.rank, w.D * w.k, std=w.gen_std)
    out["w0"] = randn(w.D, w.k, std=w.bias_std) if w.bias_std > 0 else None
    if with_dy:
        out["dy"] = randn(w.B, w.T, w.D)
    return out


def generate_proj_weight(w: Workload) -> torch.Tensor:
    """The producing projection's weight Wp[d_model, D] (for the fused form
    x = h Wp) in the I/O dtype: i.i.d. N(0, 1/d_model), so that x has about
    unit variance, from its own stream (seed + 1000) so the other inputs of
    ``w`` keep their values."""
    g = torch.Generator().manual_seed(w.seed + 1000)
    return (torch.randn(w.d, w.D, generator=g, dtype=torch.float32) * w.d ** -0.5).to(w.torch_dtype)


def moe_routing(n_seqs: int, T: int, n_experts: int, seed: int) -> list:
    """Top-1 routing counts for an MoE layer: counts[b][e] tokens of sequence
    b go to expert e, drawn with probabilities proportional to 1/(e+1) (a
    skewed load, so some experts get few or no tokens of a sequence)."""
    g = torch.Generator().manual_seed(seed)
    p = torch.tensor([1.0 / (e + 1) ** 2 for e in range(n_experts)])
    counts = []
    for _ in range(n_seqs):
        pick = torch.multinomial(p, T, replacement=True, generator=g)
        counts.append([int((pick == e).sum()) for e in range(n_experts)])
    return counts
