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

OK, E_NULL, E_SHAPE, E_K, E_DTYPE, E_ALIGN, E_ALIAS, E_WORKSPACE, E_HIP, E_LIMIT, E_SCRATCH = (
    0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10)


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
    assert dc.dynconv_abi_version() == dc.ABI_VERSION == 3
    for code in (OK, E_NULL, E_SHAPE, E_K, E_DTYPE, E_ALIGN, E_ALIAS, E_WORKSPACE, E_HIP, E_LIMIT, E_SCRATCH):
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


def test_any_width_is_accepted(L):
    """D and d_model that are not whole 16-byte vectors are valid shapes (the
    plain per-element kernels take them): sizes are reported for them."""
    for D, d, n_heads, dt in ((100, 64, 4, dc.DYNCONV_BF16), (66, 60, 6, dc.DYNCONV_FP32),
                              (128, 60, 4, dc.DYNCONV_BF16), (33, 7, 3, dc.DYNCONV_BF16)):
        p = prob(D=D, d=d, dtype=dt)
        for g in (gen_hw(n_heads=n_heads), gen_lr(rank=5)):
            assert dc.dynconv_gen_cache_bytes(p, g) > 0, (D, d)
            assert dc.dynconv_workspace_bytes(p, g, 0) > 0, (D, d)
            assert dc.dynconv_workspace_bytes(p, g, 1) > 0, (D, d)


def test_workspace_with_cache_has_no_cache_slot(L):
    """A call that gets gen_cache needs no slot for it: the size with
    DYNCONV_WS_CACHED is smaller by at least the cache bytes."""
    C = dc.DYNCONV_WS_CACHED
    for p, g in ((prob(B=4, T=512, d=256, D=512), gen_hw(n_heads=8)),
                 (prob(B=4, T=512, d=256, D=512), gen_lr(rank=16)),
                 (prob(B=2, T=100, d=32, D=64, dtype=dc.DYNCONV_FP32), gen_lr(rank=8))):
        cache = dc.dynconv_gen_cache_bytes(p, g)
        for pass_ in (0, 1):
            full = dc.dynconv_workspace_bytes(p, g, pass_)
            cached = dc.dynconv_workspace_bytes(p, g, pass_ | C)
            assert 0 <= cached <= full - cache, (pass_, full, cached, cache)
    assert dc.dynconv_workspace_bytes(prob(), gen_hw(), 4) == 0


def test_call_checks_the_workspace_it_needs(L):
    """With a cache the forward accepts the smaller workspace; without one it
    rejects that size."""
    p, g = prob(B=4, T=512, d=256, D=512), gen_hw(n_heads=8)
    small = dc.dynconv_workspace_bytes(p, g, dc.DYNCONV_WS_CACHED)
    full = dc.dynconv_workspace_bytes(p, g, 0)
    assert small < full
    # no cache: the smaller size is refused before anything is enqueued
    assert fwd(L, p, g, cache=None, ws_bytes=small) == E_WORKSPACE
    assert bwd(L, p, g, cache=None, ws_bytes=dc.dynconv_workspace_bytes(p, g, 1 | dc.DYNCONV_WS_CACHED)) \
        == E_WORKSPACE


def test_sizes(L):
    p, g = prob(), gen_hw()
    N = 4 * 4
    assert dc.dynconv_gen_cache_bytes(p, g) == 2 * 16 * N * 4
    assert dc.dynconv_workspace_bytes(p, g, 0) >= 0
    assert dc.dynconv_workspace_bytes(p, g, 1) > 0
    assert dc.dynconv_workspace_bytes(p, g, 5) == 0
    assert dc.dynconv_workspace_bytes(prob(k=9), g, 0) == 0
    assert dc.dynconv_gen_cache_bytes(prob(), gen_lr(rank=8)) == 2 * 16 * 8 * 4


@pytest.mark.parametrize("case,expect", [
    ("null_problem", E_NULL), ("null_gen", E_NULL), ("bad_dtype", E_DTYPE), ("bad_kind", E_DTYPE),
    ("k0", E_K), ("k9", E_K), ("neg_B", E_SHAPE), ("d0", E_SHAPE), ("D_heads", E_SHAPE),
    ("D_odd_empty", OK), ("d_odd_empty", OK), ("D_odd_ws_small", E_WORKSPACE), ("rank0", E_SHAPE),
    ("rank_limit", E_LIMIT),
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
    elif case == "D_odd_empty":  # any D is accepted; no tokens, so nothing is launched
        p, g = prob(B=0, D=132), gen_hw(n_heads=4)
    elif case == "d_odd_empty":
        p = prob(B=0, d=61)
    elif case == "D_odd_ws_small":  # validated like any other shape
        p, g = prob(D=100), gen_hw(n_heads=4)
        kw["ws_bytes"] = 16
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


def fwd_na(L, p, g, h=addr(1), x=addr(2), y=addr(3), cache=None):
    return L.dynconv_fwd_noalloc(ctypes.byref(p), ctypes.byref(g), h, x, y, cache, None)


@pytest.mark.parametrize("case,expect", [
    ("null_x", E_NULL), ("align_y", E_ALIGN), ("alias_y_h", E_ALIAS), ("k9", E_K), ("empty", OK),
    ("too_big_no_cache", E_SCRATCH),
])
def test_fwd_noalloc_validation(L, case, expect):
    """dynconv_fwd_noalloc validates like dynconv_fwd on the host, and refuses
    (before enqueuing anything) a call whose workspace would not fit its
    static scratch."""
    p, g = prob(), gen_hw()
    kw = {}
    if case == "null_x":
        kw["x"] = None
    elif case == "align_y":
        kw["y"] = addr(3) + 8
    elif case == "alias_y_h":
        kw["y"] = addr(1) + 512
    elif case == "k9":
        p = prob(k=9)
    elif case == "empty":
        p = prob(B=0)
    elif case == "too_big_no_cache":
        # 32768 tokens x 256 generator values x 4 bytes of cache slot: 32 MiB
        p, g = prob(B=2, T=16384, d=2048, D=4352), gen_hw(n_heads=64)
        assert dc.dynconv_workspace_bytes(p, g, 0) > dc.NOALLOC_SCRATCH_BYTES
        assert dc.dynconv_workspace_bytes(p, g, dc.DYNCONV_WS_CACHED) <= dc.NOALLOC_SCRATCH_BYTES
        kw = dict(h=BASE, x=BASE + (1 << 30), y=BASE + (2 << 30))  # tensors this large must not overlap
    assert fwd_na(L, p, g, **kw) == expect


def fwd_pj(L, p, g, h=addr(1), Wp=addr(14), x=addr(2), y=addr(3), cache=None, ws=addr(20), ws_bytes=1 << 30):
    return L.dynconv_fwd_proj(ctypes.byref(p), ctypes.byref(g), h, Wp, x, y, cache, ws, ws_bytes, None)


@pytest.mark.parametrize("case,expect", [
    ("ok_empty", OK), ("null_Wp", E_NULL), ("align_Wp", E_ALIGN), ("null_x", E_NULL),
    ("alias_x_Wp", E_ALIAS), ("alias_x_h", E_ALIAS), ("alias_x_W", E_ALIAS), ("alias_y_Wp", E_ALIAS),
    ("alias_cache_Wp", E_ALIAS), ("alias_ws_Wp", E_ALIAS), ("ws_small", E_WORKSPACE), ("k9", E_K),
])
def test_fwd_proj_validation(L, case, expect):
    """dynconv_fwd_proj: x is an output here, so it may overlap neither the
    inputs (h, the generator weights, Wp) nor the other outputs."""
    p, g = prob(), gen_hw()
    kw = {}
    if case == "ok_empty":
        p = prob(B=0)
    elif case == "null_Wp":
        kw["Wp"] = None
    elif case == "align_Wp":
        kw["Wp"] = addr(14) + 4
    elif case == "null_x":
        kw["x"] = None
    elif case == "alias_x_Wp":
        kw["x"] = addr(14) + 256
    elif case == "alias_x_h":
        kw["x"] = addr(1) + 256
    elif case == "alias_x_W":
        kw["x"] = addr(10)
    elif case == "alias_y_Wp":
        kw["y"] = addr(14)
    elif case == "alias_cache_Wp":
        kw["cache"] = addr(14) + 512
    elif case == "alias_ws_Wp":
        kw["ws"] = addr(14) - 256
    elif case == "ws_small":
        kw["ws_bytes"] = 16
    elif case == "k9":
        p = prob(k=9)
    assert fwd_pj(L, p, g, **kw) == expect


def packed(B=1, T=64, n_seqs=3, cu=addr(30), **kw):
    p = prob(B=B, T=T, **kw)
    p.cu_seqlens = cu
    p.n_seqs = n_seqs
    return p


@pytest.mark.parametrize("case,expect", [
    ("B2", E_SHAPE), ("n0", E_SHAPE), ("align", E_ALIGN), ("alias_y_cu", E_ALIAS), ("empty", OK),
    ("ws_small", E_WORKSPACE),
])
def test_packed_validation(L, case, expect):
    """Packed documents: one row, at least one document, a 4-byte aligned
    offset array that no output overlaps."""
    p, g = packed(), gen_hw()
    kw = {}
    if case == "B2":
        p = packed(B=2)
    elif case == "n0":
        p = packed(n_seqs=0)
    elif case == "align":
        p = packed(cu=addr(30) + 2)
    elif case == "alias_y_cu":
        p = packed(cu=addr(3) + 64)
    elif case == "empty":
        p = packed(T=0)
    elif case == "ws_small":
        kw["ws_bytes"] = dc.dynconv_workspace_bytes(prob(B=1, T=64), g, 0)  # the size without the position table
    assert fwd(L, p, g, **kw) == expect
    if case in ("B2", "n0", "align"):
        assert bwd(L, p, g) == expect
    if case == "alias_y_cu":  # the backward's dx over the offsets
        assert bwd(L, packed(cu=addr(4) + 64), g) == E_ALIAS


def test_packed_workspace_holds_the_position_table(L):
    """Packing adds a per-token position table (2 bytes a token) to both passes."""
    g = gen_lr()
    for pass_ in (0, 1, 2, 3):
        plain = dc.dynconv_workspace_bytes(prob(B=1, T=1000), g, pass_)
        pk = dc.dynconv_workspace_bytes(packed(T=1000), g, pass_)
        assert pk >= plain + 2 * 1000, pass_


def test_decode_refuses_packing(L):
    assert dec(L, packed(T=1), gen_hw()) == E_SHAPE


def gen_static(w0=True):
    return Gen(dc.DYNCONV_STATIC, 0, 0, 0, None, None, None, addr(13) if w0 else None)


@pytest.mark.parametrize("case,expect", [
    ("fwd_no_w0", E_NULL), ("fwd_empty", OK), ("fwd_h_null_ws_small", E_WORKSPACE), ("fwd_d_neg", E_SHAPE),
    ("fwd_w0_align", E_ALIGN), ("bwd_no_gen_grads_ws_small", E_WORKSPACE), ("bwd_no_w0", E_NULL),
    ("dec_empty", OK), ("dec_no_state", E_NULL), ("proj_h_null", E_NULL), ("kind3", E_DTYPE),
])
def test_static_validation(L, case, expect):
    """The static filter (no generator): h and the generator weights are not
    needed (d_model may be 0), w0 is; the cache holds 0 bytes."""
    p, g = prob(d=0), gen_static()
    if case == "fwd_no_w0":
        rc = fwd(L, p, gen_static(w0=False), h=None)
    elif case == "fwd_empty":
        rc = fwd(L, prob(B=0, d=0), g, h=None)
    elif case == "fwd_h_null_ws_small":
        rc = fwd(L, p, g, h=None, ws_bytes=16)
    elif case == "fwd_d_neg":
        rc = fwd(L, prob(d=-1), g, h=None)
    elif case == "fwd_w0_align":
        g.w0 = addr(13) + 8
        rc = fwd(L, p, g, h=None)
    elif case == "bwd_no_gen_grads_ws_small":
        rc = bwd(L, p, g, h=None, dh=None, gg=GenGrad(None, None, None, addr(9)), ws_bytes=16)
    elif case == "bwd_no_w0":
        rc = bwd(L, p, gen_static(w0=False), h=None, dh=None, gg=GenGrad(None, None, None, addr(9)))
    elif case == "dec_empty":
        rc = L.dynconv_decode(ctypes.byref(prob(B=0, T=1, d=0)), ctypes.byref(g), None, addr(2), addr(4),
                              addr(3), None)
    elif case == "dec_no_state":
        rc = L.dynconv_decode(ctypes.byref(prob(B=2, T=1, d=0)), ctypes.byref(g), None, addr(2), None,
                              addr(3), None)
    elif case == "proj_h_null":
        rc = fwd_pj(L, prob(d=64), g, h=None)
    else:
        g.kind = 3
        rc = fwd(L, p, g)
    assert rc == expect


def test_static_sizes(L):
    p, g = prob(d=0), gen_static()
    assert dc.dynconv_gen_cache_bytes(p, g) == 0
    assert dc.dynconv_workspace_bytes(p, g, 0) >= 4 * p.k  # the k zero generator values
    assert dc.dynconv_workspace_bytes(p, g, 1) > 0


def test_large_batches_run_in_chunks_of_sequences(L):
    """A batch whose tensors exceed the tuned kernels' 2 GiB offset limit runs
    as chunks of whole sequences: the workspace is that of the largest chunk
    (15 sequences of the Mamba-2 shape, the most whose x stays below 2 GiB),
    whatever the batch up to the boundary's own limit (2^31 elements per
    tensor: 30 sequences); batches that fit run whole."""
    def ws(B, pass_):
        return dc.dynconv_workspace_bytes(prob(B=B, T=16384, d=2048, D=4352), gen_hw(n_heads=64), pass_)
    for pass_ in (0, 1, 1 | dc.DYNCONV_WS_CACHED):
        assert 15 * 16384 * 4352 * 2 < (1 << 31) - 64 < 16 * 16384 * 4352 * 2
        assert ws(16, pass_) == ws(15, pass_) == ws(30, pass_), pass_
        assert ws(31, pass_) == 0, pass_  # beyond 2^31 elements per tensor
        assert ws(2, pass_) < ws(15, pass_), pass_
    # a packed row is never split: planned whole (here on the plain kernels:
    # the cache slot and the fp32 generator gradient, B*T*N*4 bytes each, and
    # the position table)
    p = packed(T=16 * 16384, D=4352, d=2048)
    BT, N = 16 * 16384, 256
    assert dc.dynconv_workspace_bytes(p, gen_hw(n_heads=64), 1) >= 2 * BT * N * 4 + BT * 2


@pytest.mark.parametrize("B,T", [(0, 300), (3, 0), (0, 0)])
def test_empty_batch_sizes(L, B, T):
    """Workspace sizes of empty batches for every kind, width and dtype: the
    layouts of the tuned kernels keep at least one tile per token range (an
    empty batch once divided by a zero tile count there)."""
    for D in (64, 200, 360, 4352):
        for dt in (dc.DYNCONV_BF16, dc.DYNCONV_FP32):
            gens = [gen_lr(rank=r) for r in (1, 16, 33, 64)] + [gen_static()]
            gens += [gen_hw(n_heads=h) for h in (1, 8, 64) if D % h == 0]
            for g in gens:
                for pass_ in (0, 1, 1 | dc.DYNCONV_WS_CACHED):
                    assert dc.dynconv_workspace_bytes(prob(B=B, T=T, d=128, D=D, k=4, dtype=dt), g, pass_) >= 0
