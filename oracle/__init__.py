"""fp64 CPU oracle of the dynamic short convolution layer (forward + backward).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the GPU library under ``input_dependent_depthwise_amd/`` and neither
side imports the other.

The arithmetic lives in ``dynconv_oracle.c`` (plain loops in fp64, OpenMP over
independent outputs, built with gcc and no fast-math); this module only
marshals numpy arrays into it.  What it computes follows "Dynamic Short
Convolutions Improve Transformers" (gist.science Technical Summary,
Methodology -> Dynamic Short Convolutions: Mechanism, Parameterization,
Placement; Efficient Training Implementation -> Fused Low-Rank Kernel).  The
formulas are restated in the C file's header.

Pins (tests/test_oracle_pins.py): hand-worked examples in tests/golden/, the
static special case against torch conv1d, a dense-matrix formulation, torch
autograd gradients, central finite differences, the adjoint identity,
causality, batch isolation, head-wise == low-rank equivalence and linearity.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dynconv_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

HEADWISE = 0
LOWRANK = 1


def build(force: bool = True) -> str:
    """Compile the C oracle into ``oracle/liboracle.so`` (gcc, -O2, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-Wall", "-Werror", "-o", tmp, _SRC]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("d", ctypes.c_int64),
                ("D", ctypes.c_int64), ("k", ctypes.c_int32), ("kind", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("doc", ctypes.POINTER(ctypes.c_int64))]


class OracleLib:
    """The oracle's C library.  ``path`` defaults to ``oracle/liboracle.so``;
    the mutation tests load deliberately broken copies through it."""

    def __init__(self, path: str | None = None):
        if path is None:
            if not os.path.exists(_LIB):
                build(force=False)
            path = _LIB
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        lib.orc_filters.argtypes = [ctypes.POINTER(_Shape)] + [P] * 7
        lib.orc_conv.argtypes = [ctypes.POINTER(_Shape), P, P, P]
        lib.orc_backward.argtypes = [ctypes.POINTER(_Shape)] + [P] * 13
        lib.orc_proj.argtypes = [ctypes.POINTER(_Shape), P, P, P]
        for f in (lib.orc_filters, lib.orc_conv, lib.orc_backward, lib.orc_proj):
            f.restype = ctypes.c_int
        lib.orc_num_threads.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def num_threads(self) -> int:
        """OpenMP threads the oracle runs on."""
        return int(self.lib.orc_num_threads())

    def proj(self, s: "Shape", h, Wp):
        """The producing projection x = h Wp ([B*T, D], float64)."""
        cs = s._c()
        h = _f64(h, (s.B * s.T, s.d))
        Wp = _f64(Wp, (s.d, s.D))
        x = np.empty((s.B * s.T, s.D), dtype=np.float64)
        _check(self.lib.orc_proj(ctypes.byref(cs), _p(h), _p(Wp), _p(x)), "proj")
        return x

    def filters(self, s: "Shape", h, W=None, A=None, U=None, w0=None):
        """Steps 1-2: returns (w[B*T, D, k], gen) with gen = u or z ([B*T, N])."""
        BT = s.B * s.T
        h = _f64(h, (BT, s.d))
        W = _f64(W, (s.d, s.n_heads * s.k)) if s.kind == HEADWISE else None
        A = _f64(A, (s.d, s.rank)) if s.kind == LOWRANK else None
        U = _f64(U, (s.rank, s.D * s.k)) if s.kind == LOWRANK else None
        w0 = _f64(w0, (s.D, s.k))
        w = np.empty((BT, s.D, s.k), dtype=np.float64)
        gen = np.empty((BT, s.gen_cols), dtype=np.float64)
        cs = s._c()
        _check(self.lib.orc_filters(ctypes.byref(cs), _p(h), _p(W), _p(A), _p(U), _p(w0),
                                    _p(w), _p(gen)), "filters")
        return w, gen

    def conv(self, s: "Shape", w, x):
        """Step 3: y = x + causal depthwise conv with per-token filters w."""
        BT = s.B * s.T
        w = _f64(w, (BT, s.D, s.k))
        x = _f64(x, (BT, s.D))
        y = np.empty((BT, s.D), dtype=np.float64)
        cs = s._c()
        _check(self.lib.orc_conv(ctypes.byref(cs), _p(w), _p(x), _p(y)), "conv")
        return y

    def forward(self, s: "Shape", h, x, W=None, A=None, U=None, w0=None):
        """Whole forward.  Returns dict(y, w, gen) as float64 arrays ([B*T, ...])."""
        w, gen = self.filters(s, h, W=W, A=A, U=U, w0=w0)
        y = self.conv(s, w, x)
        return {"y": y, "w": w, "gen": gen}

    def backward(self, s: "Shape", h, x, dy, W=None, A=None, U=None, w0=None, w=None):
        """Whole backward for L = sum(dy * y).

        Returns dict(dx, dh, dw0, and dW (head-wise) or dA, dU (low-rank)),
        float64.  ``w`` (the forward filters) is recomputed when not given.
        """
        BT = s.B * s.T
        if w is None:
            w, _ = self.filters(s, h, W=W, A=A, U=U, w0=w0)
        h = _f64(h, (BT, s.d))
        x = _f64(x, (BT, s.D))
        dy = _f64(dy, (BT, s.D))
        w = _f64(w, (BT, s.D, s.k))
        Wd = _f64(W, (s.d, s.n_heads * s.k)) if s.kind == HEADWISE else None
        Ad = _f64(A, (s.d, s.rank)) if s.kind == LOWRANK else None
        Ud = _f64(U, (s.rank, s.D * s.k)) if s.kind == LOWRANK else None
        out = {"dx": np.empty((BT, s.D)), "dh": np.empty((BT, s.d)), "dw0": np.empty((s.D, s.k))}
        if s.kind == HEADWISE:
            out["dW"] = np.empty((s.d, s.n_heads * s.k))
            dW, dA, dU = out["dW"], None, None
        else:
            out["dA"] = np.empty((s.d, s.rank))
            out["dU"] = np.empty((s.rank, s.D * s.k))
            dW, dA, dU = None, out["dA"], out["dU"]
        cs = s._c()
        _check(self.lib.orc_backward(ctypes.byref(cs), _p(h), _p(Wd), _p(Ad), _p(Ud), _p(x), _p(w),
                                     _p(dy), _p(out["dx"]), _p(out["dh"]), _p(dW), _p(dA), _p(dU),
                                     _p(out["dw0"])), "backward")
        return out


_default = None


def default() -> OracleLib:
    global _default
    if _default is None:
        _default = OracleLib()
    return _default


@dataclass(frozen=True)
class Shape:
    B: int
    T: int
    d: int
    D: int
    k: int
    kind: int          # HEADWISE or LOWRANK
    n_heads: int = 0
    rank: int = 0
    # packed documents: offsets 0 = c_0 <= c_1 <= ... <= c_n = B*T of the
    # documents in the flattened tokens (None: one document per batch row)
    cu_seqlens: tuple | None = None

    def doc_index(self):
        """Document index of every token ([B*T] int64), or None."""
        if self.cu_seqlens is None:
            return None
        cu = [int(c) for c in self.cu_seqlens]
        if cu[0] != 0 or cu[-1] != self.B * self.T or any(b < a for a, b in zip(cu, cu[1:])):
            raise ValueError(f"cu_seqlens must rise from 0 to B*T = {self.B * self.T}: {cu}")
        doc = np.empty(self.B * self.T, dtype=np.int64)
        for i in range(len(cu) - 1):
            doc[cu[i]:cu[i + 1]] = i
        return doc

    def _c(self) -> _Shape:
        c = _Shape(self.B, self.T, self.d, self.D, self.k, self.kind, self.n_heads, self.rank, None)
        doc = self.doc_index()
        if doc is not None:
            c._doc = doc  # keeps the array alive as long as the struct
            c.doc = doc.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
        return c

    @property
    def gen_cols(self) -> int:
        return self.n_heads * self.k if self.kind == HEADWISE else self.rank


def _f64(a, shape=None):
    """Contiguous float64 copy (exact widening of fp32 / bf16 values)."""
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor
        a = a.detach().to("cpu").double().numpy()
    a = np.ascontiguousarray(a, dtype=np.float64)
    if shape is not None:
        a = a.reshape(shape)
    return a


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (code {rc})")


def num_threads() -> int:
    return default().num_threads()


def proj(s: Shape, h, Wp):
    return default().proj(s, h, Wp)


def filters(s: Shape, h, W=None, A=None, U=None, w0=None):
    return default().filters(s, h, W=W, A=A, U=U, w0=w0)


def conv(s: Shape, w, x):
    return default().conv(s, w, x)


def forward(s: Shape, h, x, W=None, A=None, U=None, w0=None):
    return default().forward(s, h, x, W=W, A=A, U=U, w0=w0)


def backward(s: Shape, h, x, dy, W=None, A=None, U=None, w0=None, w=None):
    return default().backward(s, h, x, dy, W=W, A=A, U=U, w0=w0, w=w)
