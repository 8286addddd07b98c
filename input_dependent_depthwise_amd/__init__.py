"""MI355X (gfx950) dynamic short convolution: Python binding of libdynconv.

Thin ctypes binding of the C ABI in ``include/dynconv.h``, with the same
names (``dynconv_fwd``, ``dynconv_bwd``, ``dynconv_decode``, ``dynconv_workspace_bytes``,
``dynconv_gen_cache_bytes``, ``dynconv_status_str``, ``dynconv_abi_version``).
It only marshals arguments: torch provides device memory (outputs and
workspace are ``torch.empty``) and the current HIP stream; every step of the
layer runs in the library's HIP kernels.  There is no CPU fallback: if the
library is not built this module raises on import of the binding.

The layer ("Dynamic Short Convolutions Improve Transformers", gist.science
Technical Summary, Methodology -> Dynamic Short Convolutions) is
``y = x + sum_j w_t[:, j] * x_{t-j}`` with the per-token filter ``w_t``
generated from the hidden state ``h_t`` head-wise (``W``) or low-rank
(``A``, ``U``), plus a static bias ``w0``.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdynconv.so")

DYNCONV_FP32, DYNCONV_BF16 = 0, 1
DYNCONV_HEADWISE, DYNCONV_LOWRANK, DYNCONV_STATIC = 0, 1, 2
ABI_VERSION = 3
DYNCONV_WS_CACHED = 2  # or-ed into dynconv_workspace_bytes' pass when the call gets gen_cache


class DynConvError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {dynconv_status_str(status)} (status {status})")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("d_model", ctypes.c_int64),
                ("D", ctypes.c_int64), ("k", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("cu_seqlens", ctypes.c_void_p), ("n_seqs", ctypes.c_int64)]


class Gen(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("W", ctypes.c_void_p), ("A", ctypes.c_void_p),
                ("U", ctypes.c_void_p), ("w0", ctypes.c_void_p)]


class GenGrad(ctypes.Structure):
    _fields_ = [("dW", ctypes.c_void_p), ("dA", ctypes.c_void_p), ("dU", ctypes.c_void_p),
                ("dw0", ctypes.c_void_p)]


# names the C header declares; the CPU tests check each is exported
EXPORTS = ("dynconv_fwd", "dynconv_fwd_proj", "dynconv_fwd_noalloc", "dynconv_bwd", "dynconv_decode", "dynconv_workspace_bytes",
           "dynconv_gen_cache_bytes", "dynconv_status_str", "dynconv_abi_version", "dynconv_trace_next")
DYNCONV_E_SCRATCH = -10
NOALLOC_SCRATCH_BYTES = 16 << 20  # the static scratch of dynconv_fwd_noalloc

# kernel ids for dynconv_trace_next
DYNCONV_K_GEN_PROJ, DYNCONV_K_FWD_CONV, DYNCONV_K_BWD_CONV, DYNCONV_K_GEN_BWD, DYNCONV_K_FINALIZE = 1, 2, 3, 4, 5

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libdynconv.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m input_dependent_depthwise_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        PP, PG, PGG = ctypes.POINTER(Problem), ctypes.POINTER(Gen), ctypes.POINTER(GenGrad)
        L.dynconv_fwd.argtypes = [PP, PG, P, P, P, P, P, ctypes.c_size_t, P]
        L.dynconv_fwd.restype = ctypes.c_int
        L.dynconv_fwd_proj.argtypes = [PP, PG, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.dynconv_fwd_proj.restype = ctypes.c_int
        L.dynconv_fwd_noalloc.argtypes = [PP, PG, P, P, P, P, P]
        L.dynconv_fwd_noalloc.restype = ctypes.c_int
        L.dynconv_bwd.argtypes = [PP, PG, P, P, P, P, P, P, PGG, P, ctypes.c_size_t, P]
        L.dynconv_bwd.restype = ctypes.c_int
        L.dynconv_decode.argtypes = [PP, PG, P, P, P, P, P]
        L.dynconv_decode.restype = ctypes.c_int
        L.dynconv_workspace_bytes.argtypes = [PP, PG, ctypes.c_int]
        L.dynconv_workspace_bytes.restype = ctypes.c_size_t
        L.dynconv_gen_cache_bytes.argtypes = [PP, PG]
        L.dynconv_gen_cache_bytes.restype = ctypes.c_size_t
        L.dynconv_status_str.argtypes = [ctypes.c_int]
        L.dynconv_status_str.restype = ctypes.c_char_p
        L.dynconv_abi_version.restype = ctypes.c_int
        L.dynconv_trace_next.argtypes = [ctypes.c_int, P, P]
        L.dynconv_trace_next.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _dtype_code(dt) -> int:
    if dt == torch.float32:
        return DYNCONV_FP32
    if dt == torch.bfloat16:
        return DYNCONV_BF16
    raise TypeError(f"unsupported I/O dtype {dt}")


def make_problem(x: torch.Tensor, h, k: int, cu_seqlens=None) -> Problem:
    """Problem struct from x[B,T,D], h[B,T,d_model] and the filter width k.

    h may be None for the static filter (d_model 0).  cu_seqlens: None, or
    packed documents (B must be 1): an int32 device tensor of n_seqs + 1
    offsets rising from 0 to T."""
    if x.dim() != 3 or (h is not None and (h.dim() != 3 or h.shape[:2] != x.shape[:2])):
        raise ValueError(f"expected h[B,T,d] and x[B,T,D], got {None if h is None else tuple(h.shape)} "
                         f"and {tuple(x.shape)}")
    B, T, D = x.shape
    d = 0 if h is None else h.shape[2]
    if cu_seqlens is None:
        return Problem(B, T, d, D, int(k), _dtype_code(x.dtype), None, 0)
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
        raise TypeError("cu_seqlens must be a contiguous 1-d int32 tensor")
    return Problem(B, T, d, D, int(k), _dtype_code(x.dtype), cu_seqlens.data_ptr(), cu_seqlens.numel() - 1)


def make_gen(W=None, A=None, U=None, w0=None, n_heads: int = 0) -> Gen:
    """Generator struct: head-wise when W is given, low-rank when A and U
    are, the static filter (w0 alone) when none of them is."""
    if W is None and A is None and U is None:
        if w0 is None:
            raise ValueError("the static filter needs w0")
        return Gen(DYNCONV_STATIC, 0, 0, 0, None, None, None, _ptr(w0))
    if W is not None:
        if n_heads <= 0:
            raise ValueError("head-wise generator needs n_heads")
        return Gen(DYNCONV_HEADWISE, int(n_heads), 0, 0, _ptr(W), None, None, _ptr(w0))
    if A is None or U is None:
        raise ValueError("pass W (head-wise) or both A and U (low-rank)")
    return Gen(DYNCONV_LOWRANK, 0, int(A.shape[1]), 0, None, _ptr(A), _ptr(U), _ptr(w0))


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(rc: int, where: str):
    if rc != 0:
        raise DynConvError(rc, where)


def dynconv_status_str(status: int) -> str:
    return lib().dynconv_status_str(int(status)).decode()


def dynconv_abi_version() -> int:
    return int(lib().dynconv_abi_version())


def dynconv_trace_next(kernel: int, start, stop) -> None:
    """Arm a one-shot event pair around the next launch of ``kernel`` on this
    thread (torch.cuda.Event objects, or None to disarm)."""
    a = None if start is None else start.cuda_event
    b = None if stop is None else stop.cuda_event
    _check(lib().dynconv_trace_next(int(kernel), a, b), "dynconv_trace_next")


def dynconv_workspace_bytes(prob: Problem, gen: Gen, pass_: int) -> int:
    return int(lib().dynconv_workspace_bytes(ctypes.byref(prob), ctypes.byref(gen), int(pass_)))


def dynconv_gen_cache_bytes(prob: Problem, gen: Gen) -> int:
    return int(lib().dynconv_gen_cache_bytes(ctypes.byref(prob), ctypes.byref(gen)))


def _workspace(nbytes: int, device, workspace):
    if workspace is not None:
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def dynconv_fwd(h, x, *, k, W=None, A=None, U=None, w0=None, n_heads=0, y=None, gen_cache=None,
                want_cache=False, workspace=None, stream=None, cu_seqlens=None):
    """Forward: returns y (and the fp32 generator cache when want_cache).
    cu_seqlens: packed documents in a single row (see make_problem)."""
    prob = make_problem(x, h, k, cu_seqlens)
    gen = make_gen(W, A, U, w0, n_heads)
    if y is None:
        y = torch.empty_like(x)
    if gen_cache is None and want_cache and gen.kind != DYNCONV_STATIC:
        n = gen.n_heads * k if gen.kind == DYNCONV_HEADWISE else gen.rank
        gen_cache = torch.empty(x.shape[0] * x.shape[1], n, dtype=torch.float32, device=x.device)
    nbytes = dynconv_workspace_bytes(prob, gen, 0 | (DYNCONV_WS_CACHED if gen_cache is not None else 0))
    ws = _workspace(nbytes, x.device, workspace)
    rc = lib().dynconv_fwd(ctypes.byref(prob), ctypes.byref(gen), _ptr(h), _ptr(x), _ptr(y),
                           _ptr(gen_cache), _ptr(ws), ws.numel() * ws.element_size(),
                           _stream(stream))
    _check(rc, "dynconv_fwd")
    return (y, gen_cache) if want_cache else y


def dynconv_fwd_proj(h, Wp, *, k, W=None, A=None, U=None, w0=None, n_heads=0, x=None, y=None, gen_cache=None,
                     want_cache=False, workspace=None, stream=None, cu_seqlens=None):
    """Forward with the producing projection fused in: x = h Wp, then
    y = x + dynconv(x).  Returns (x, y) (and the generator cache when
    want_cache)."""
    B, T = h.shape[0], h.shape[1]
    if x is None:
        x = torch.empty(B, T, Wp.shape[1], dtype=h.dtype, device=h.device)
    prob = make_problem(x, h, k, cu_seqlens)
    gen = make_gen(W, A, U, w0, n_heads)
    if y is None:
        y = torch.empty_like(x)
    if gen_cache is None and want_cache and gen.kind != DYNCONV_STATIC:
        n = gen.n_heads * k if gen.kind == DYNCONV_HEADWISE else gen.rank
        gen_cache = torch.empty(B * T, n, dtype=torch.float32, device=h.device)
    nbytes = dynconv_workspace_bytes(prob, gen, 0 | (DYNCONV_WS_CACHED if gen_cache is not None else 0))
    ws = _workspace(nbytes, h.device, workspace)
    rc = lib().dynconv_fwd_proj(ctypes.byref(prob), ctypes.byref(gen), _ptr(h), _ptr(Wp), _ptr(x), _ptr(y),
                                _ptr(gen_cache), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "dynconv_fwd_proj")
    return (x, y, gen_cache) if want_cache else (x, y)


def dynconv_fwd_noalloc(h, x, *, k, W=None, A=None, U=None, w0=None, n_heads=0, y=None, gen_cache=None,
                        stream=None, cu_seqlens=None):
    """Forward whose workspace is the library's static scratch (no workspace
    argument).  y and gen_cache, when not given, are allocated here by torch,
    outside the library call; pass them for a call that allocates nothing."""
    prob = make_problem(x, h, k, cu_seqlens)
    gen = make_gen(W, A, U, w0, n_heads)
    if y is None:
        y = torch.empty_like(x)
    rc = lib().dynconv_fwd_noalloc(ctypes.byref(prob), ctypes.byref(gen), _ptr(h), _ptr(x), _ptr(y),
                                   _ptr(gen_cache), _stream(stream))
    _check(rc, "dynconv_fwd_noalloc")
    return y


def dynconv_bwd(h, x, dy, *, k, W=None, A=None, U=None, w0=None, n_heads=0, gen_cache=None,
                need_dh=True, need_dw0=True, out=None, workspace=None, stream=None, cu_seqlens=None):
    """Backward of sum(dy * y).  Returns dict(dx, dh, dw0, dW | dA, dU).
    cu_seqlens: packed documents, as given to the forward."""
    prob = make_problem(x, h, k, cu_seqlens)
    gen = make_gen(W, A, U, w0, n_heads)
    dev = x.device
    f32 = dict(dtype=torch.float32, device=dev)
    o = dict(out or {})
    o.setdefault("dx", torch.empty_like(x))
    if need_dh and h is not None:
        o.setdefault("dh", torch.empty_like(h))
    if need_dw0:
        o.setdefault("dw0", torch.empty(prob.D, k, **f32))
    if gen.kind == DYNCONV_STATIC:
        pass
    elif gen.kind == DYNCONV_HEADWISE:
        o.setdefault("dW", torch.empty(prob.d_model, gen.n_heads * k, **f32))
    else:
        o.setdefault("dA", torch.empty(prob.d_model, gen.rank, **f32))
        o.setdefault("dU", torch.empty(gen.rank, prob.D * k, **f32))
    gg = GenGrad(_ptr(o.get("dW")), _ptr(o.get("dA")), _ptr(o.get("dU")), _ptr(o.get("dw0")))
    nbytes = dynconv_workspace_bytes(prob, gen, 1 | (DYNCONV_WS_CACHED if gen_cache is not None else 0))
    ws = _workspace(nbytes, dev, workspace)
    rc = lib().dynconv_bwd(ctypes.byref(prob), ctypes.byref(gen), _ptr(h), _ptr(x), _ptr(dy),
                           _ptr(gen_cache), _ptr(o["dx"]), _ptr(o.get("dh")), ctypes.byref(gg),
                           _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "dynconv_bwd")
    return o


def dynconv_decode(h, x, state, *, k, W=None, A=None, U=None, w0=None, n_heads=0, y=None, stream=None):
    """One decoding step: h [B, d_model], x [B, D], state [B, k-1, D] (updated
    in place; None when k == 1).  Returns y [B, D]."""
    B, D = x.shape
    prob = Problem(B, 1, 0 if h is None else h.shape[-1], D, k, _dtype_code(x.dtype), None, 0)
    gen = make_gen(W, A, U, w0, n_heads)
    if y is None:
        y = torch.empty_like(x)
    rc = lib().dynconv_decode(ctypes.byref(prob), ctypes.byref(gen), _ptr(h), _ptr(x), _ptr(state), _ptr(y),
                              _stream(stream))
    _check(rc, "dynconv_decode")
    return y


class DynConvFn(torch.autograd.Function):
    """autograd wrapper: y = DynConvFn.apply(h, x, W, A, U, w0, k, n_heads[, cu_seqlens]).

    Pass W (head-wise, with n_heads) or A and U (low-rank), or none of them
    for the static filter (w0 alone; h may then be None); unused weights are
    None; cu_seqlens packs documents into one row.  The forward keeps the
    fp32 generator cache for the backward.
    """

    @staticmethod
    def forward(ctx, h, x, W, A, U, w0, k, n_heads, cu_seqlens=None):
        y, cache = dynconv_fwd(h, x, k=k, W=W, A=A, U=U, w0=w0, n_heads=n_heads, want_cache=True,
                               cu_seqlens=cu_seqlens)
        ctx.save_for_backward(h, x, W, A, U, w0, cache, cu_seqlens)
        ctx.k, ctx.n_heads = k, n_heads
        return y

    @staticmethod
    def backward(ctx, dy):
        h, x, W, A, U, w0, cache, cu_seqlens = ctx.saved_tensors
        g = dynconv_bwd(h, x, dy.contiguous(), k=ctx.k, W=W, A=A, U=U, w0=w0, n_heads=ctx.n_heads,
                        gen_cache=cache, need_dh=ctx.needs_input_grad[0],
                        need_dw0=w0 is not None, cu_seqlens=cu_seqlens)
        cast = lambda t, ref: None if t is None or ref is None else t.to(ref.dtype)
        return (g.get("dh"), g["dx"], cast(g.get("dW"), W), cast(g.get("dA"), A),
                cast(g.get("dU"), U), cast(g.get("dw0"), w0), None, None, None)
