"""C-ABI checks that need no GPU: the library loads, exports every function
include/dynconv.h declares, sizes its workspace, and rejects bad arguments on
the host (fake, never-dereferenced device addresses; no kernel is launched).
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import input_dependent_depthwise_amd as dc
from input_dependent_depthwise_amd import Gen, GenGrad, Problem

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dynconv.h")

OK, E_NULL, E_SHAPE, E_K, E_DTYPE, E_ALIGN, E_ALIAS, E_WORKSPACE, E_HIP, E_LIMIT = (
    0, -1, -2, -3, -4, -5, -6, -7, -8, -9)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(dc.LIB_PATH):
        from input_dependent_depthwise_amd import build
        build.build()
    return dc.lib()


def header_functions():
    text = open(HEADER).read()
    return re.findall(r"DYNCONV_API\s+[\w\s\*]+?\b(dynconv_\w+)\s*\(", text)


def test_header_declares_the_binding_names():
    assert sorted(header_functions()) == sorted(dc.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    for name in header_functions():
        assert hasattr(L, name), name


def test_version_and_status_strings(L):
    assert dc.dynconv_abi_version() == 1
    for code in (OK, E_NULL, E_SHAPE, E_K, E_DTYPE, E_ALIGN, E_ALIAS, E_WORKSPACE, E_HIP, E_LIMIT):
        s = dc.dynconv_status_str(code)
        assert s and s != "unknown status"
    assert dc.dynconv_status_str(-1234) == "unknown status"


# fake device addresses: 1 MiB apart, 256-byte aligned, never dereferenced
BASE = 1 << 40
MB = 1 << 20


def addr(i):
    return BASE + i * 64 * MB


def prob(B=2, T=16, d=64, D=128, k=4, dtype=dc.DYNCONV_BF16):
    return Problem(B, T, d, D, k, dtype)


def gen_hw(n_heads=4, w0=True):
    return Gen(dc.DYNCONV_HEADWISE, n_heads, 0, 0, addr(10), None, None, addr(13) if w0 else None)


def gen_lr(rank=16, w0=True):
    return Gen(dc.DYNCONV_LOWRANK, 0, rank, 0, None, addr(11), addr(12), addr(13) if w0 else None)


def fwd(L, p, g, h=addr(1), x=addr(2), y=addr(3), cache=None, ws=addr(20), ws_bytes=1 << 30):
    return L.dynconv_fwd(ctypes.byref(p) if p is not None else None,
                         ctypes.byref(g) if g is not None else None, h, x, y, cache, ws, ws_bytes,
                         None)


def bwd(L, p, g, h=addr(1), x=addr(2), dy=addr(3), cache=None, dx=addr(4), dh=addr(5),
        gg=None, ws=addr(20), ws_bytes=1 << 30):
    if gg is None:
        gg = GenGrad(addr(6), addr(7), addr(8), addr(9))
    return L.dynconv_bwd(ctypes.byref(p), ctypes.byref(g), h, x, dy, cache, dx, dh, ctypes.byref(gg),
                         ws, ws_bytes, None)


def test_sizes(L):
    p, g = prob(), gen_hw()
    N = 4 * 4
    assert dc.dynconv_gen_cache_bytes(p, g) == 2 * 16 * N * 4
    assert dc.dynconv_workspace_bytes(p, g, 0) >= 0
    assert dc.dynconv_workspace_bytes(p, g, 1) > 0
    assert dc.dynconv_workspace_bytes(p, g, 2) == 0
    assert dc.dynconv_workspace_bytes(prob(k=9), g, 0) == 0
    assert dc.dynconv_gen_cache_bytes(prob(), gen_lr(rank=8)) == 2 * 16 * 8 * 4


@pytest.mark.parametrize("case,expect", [
    ("null_problem", E_NULL), ("null_gen", E_NULL), ("bad_dtype", E_DTYPE), ("bad_kind", E_DTYPE),
    ("k0", E_K), ("k9", E_K), ("neg_B", E_SHAPE), ("d0", E_SHAPE), ("D_heads", E_SHAPE),
    ("D_vec", E_SHAPE), ("d_vec", E_SHAPE), ("rank0", E_SHAPE), ("rank_limit", E_LIMIT),
    ("heads_limit", E_LIMIT), ("null_h", E_NULL), ("null_W", E_NULL), ("null_U", E_NULL),
    ("align_x", E_ALIGN), ("align_w0", E_ALIGN), ("alias_y_x", E_ALIAS),
    ("alias_cache_h", E_ALIAS), ("alias_ws_y", E_ALIAS), ("ws_small", E_WORKSPACE),
    ("ws_null", E_WORKSPACE), ("empty", OK), ("big", E_LIMIT),
])
def test_fwd_validation(L, case, expect):
    p, g = prob(), gen_hw()
    kw = {}
    if case == "null_problem":
        p = None
    elif case == "null_gen":
        g = None
    elif case == "bad_dtype":
        p = prob(dtype=7)
    elif case == "bad_kind":
        g.kind = 5
    elif case == "k0":
        p = prob(k=0)
    elif case == "k9":
        p = prob(k=9)
    elif case == "neg_B":
        p = prob(B=-1)
    elif case == "d0":
        p = prob(d=0)
    elif case == "D_heads":
        g = gen_hw(n_heads=3)
    elif case == "D_vec":
        p, g = prob(D=132), gen_hw(n_heads=4)
    elif case == "d_vec":
        p = prob(d=60)
    elif case == "rank0":
        g = gen_lr(rank=0)
    elif case == "rank_limit":
        g = gen_lr(rank=65)
    elif case == "heads_limit":
        p, g = prob(D=1024, k=8), gen_hw(n_heads=64)
    elif case == "null_h":
        kw["h"] = None
    elif case == "null_W":
        g.W = None
    elif case == "null_U":
        g = gen_lr()
        g.U = None
    elif case == "align_x":
        kw["x"] = addr(2) + 2
    elif case == "align_w0":
        g.w0 = addr(13) + 8
    elif case == "alias_y_x":
        kw["y"] = addr(2) + 256
    elif case == "alias_cache_h":
        kw["cache"] = addr(1) + 1024
    elif case == "alias_ws_y":
        kw["ws"] = addr(3) - 256
    elif case == "ws_small":
        kw["ws_bytes"] = 16
    elif case == "ws_null":
        kw["ws"] = None
    elif case == "empty":
        p = prob(B=0)
    elif case == "big":
        p = prob(B=1 << 20, T=1 << 12)
    assert fwd(L, p, g, **kw) == expect


@pytest.mark.parametrize("case,expect", [
    ("null_gg", E_NULL), ("null_dW", E_NULL), ("null_dU", E_NULL), ("null_dy", E_NULL),
    ("null_dx", E_NULL), ("align_dh", E_ALIGN), ("alias_dx_dy", E_ALIAS),
    ("alias_dh_dx", E_ALIAS), ("alias_dW_W", E_ALIAS), ("alias_ws_cache", E_ALIAS),
    ("ws_small", E_WORKSPACE),
])
def test_bwd_validation(L, case, expect):
    p, g = prob(), gen_hw()
    kw = {}
    if case == "null_gg":
        rc = L.dynconv_bwd(ctypes.byref(p), ctypes.byref(g), addr(1), addr(2), addr(3), None,
                           addr(4), addr(5), None, addr(20), 1 << 30, None)
        assert rc == expect
        return
    if case == "null_dW":
        kw["gg"] = GenGrad(None, None, None, None)
    elif case == "null_dU":
        g = gen_lr()
        kw["gg"] = GenGrad(None, addr(7), None, addr(9))
    elif case == "null_dy":
        kw["dy"] = None
    elif case == "null_dx":
        kw["dx"] = None
    elif case == "align_dh":
        kw["dh"] = addr(5) + 4
    elif case == "alias_dx_dy":
        kw["dx"] = addr(3)
    elif case == "alias_dh_dx":
        kw["dh"] = addr(4) + 512
    elif case == "alias_dW_W":
        kw["gg"] = GenGrad(addr(10), None, None, addr(9))
    elif case == "alias_ws_cache":
        kw["cache"] = addr(21)
        kw["ws"] = addr(21) - 1024
    elif case == "ws_small":
        kw["ws_bytes"] = 100
    assert bwd(L, p, g, **kw) == expect


def dec(L, p, g, h=addr(1), x=addr(2), state=addr(3), y=addr(4)):
    return L.dynconv_decode(ctypes.byref(p) if p is not None else None,
                            ctypes.byref(g) if g is not None else None, h, x, state, y, None)


@pytest.mark.parametrize("case,expect", [
    ("null_problem", E_NULL), ("T2", E_SHAPE), ("k9", E_K), ("null_x", E_NULL), ("null_state", E_NULL),
    ("null_W", E_NULL), ("align_y", E_ALIGN), ("alias_y_state", E_ALIAS), ("alias_state_x", E_ALIAS),
    ("B_limit", E_LIMIT), ("empty", OK),
])
def test_decode_validation(L, case, expect):
    """dynconv_decode rejects bad arguments on the host; B == 0 is a no-op."""
    p, g = prob(T=1), gen_hw()
    kw = {}
    if case == "null_problem":
        p = None
    elif case == "T2":
        p = prob(T=2)
    elif case == "k9":
        p = prob(T=1, k=9)
    elif case == "null_x":
        kw["x"] = None
    elif case == "null_state":
        kw["state"] = None
    elif case == "null_W":
        g.W = None
    elif case == "align_y":
        kw["y"] = addr(4) + 4
    elif case == "alias_y_state":
        kw["y"] = addr(3) + 256
    elif case == "alias_state_x":
        kw["state"] = addr(2)
    elif case == "B_limit":
        p = prob(B=70000, T=1)
    elif case == "empty":
        p = prob(B=0, T=1)
    assert dec(L, p, g, **kw) == expect
