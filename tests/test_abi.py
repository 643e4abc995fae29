"""The C-ABI library on the CPU: it loads, exports every symbol include/tern.h
declares, and rejects bad arguments before touching the GPU.  No call here
passes validation, so no kernel is launched."""
import ctypes
import os
import re

import pytest

import ternary_weight_linear_tern_amd as tl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tern.h")

OK, NULL, SHAPE, THETA, DTYPE, ALIGN, WORKSPACE, ALIAS = 0, -1, -2, -3, -4, -5, -6, -7
F32, BF16 = 0, 1


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tern_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(tl.LIB_PATH):
        from ternary_weight_linear_tern_amd import build
        build.build()
    return tl.lib()


def P(addr):
    return ctypes.c_void_p(addr)


def test_exports_every_declared_symbol(L):
    names = header_functions()
    assert len(names) >= 9, names
    for n in names:
        assert hasattr(L, n), f"libtern.so does not export {n}"
        assert n in tl.SIGNATURES, f"binding has no signature for {n}"


def test_status_strings(L):
    for code in range(-10, 1):
        s = tl.tern_status_str(code)
        assert s and s != "unknown status"
    assert tl.tern_status_str(-99) == "unknown status"
    assert "gfx950" in tl.tern_version()


def _layout_words(n_in, n_out):
    """The handle layout of include/tern.h: canonical words, then the forward
    and dX fragment copies (512 words per 256-row tile and 32-wide K chunk),
    the first copy starting on a 64-word boundary."""
    if n_in == 0 or n_out == 0:
        return 0
    cd = lambda a, b: -(-a // b)
    canon = n_in * cd(n_out, 16)
    return cd(canon, 64) * 64 + (cd(n_out, 256) * cd(n_in, 32) + cd(n_in, 256) * cd(n_out, 32)) * 512


def test_packed_words(L):
    assert tl.tern_packed_words(0, 0) == 0
    assert tl.tern_packed_words(0, 32) == 0
    assert tl.tern_packed_words(-1, 4) == -1
    assert tl.tern_packed_words(3, 16) == 64 + 512 + 512
    assert tl.tern_packed_words(256, 256) == 4096 + (8 + 8) * 512
    for n_in, n_out in [(3, 17), (2, 20), (136, 264), (2048, 8192), (4096, 16384)]:
        assert tl.tern_packed_words(n_in, n_out) == _layout_words(n_in, n_out), (n_in, n_out)


def test_materialize_rejects(L):
    s = P(0)
    m = L.tern_materialize
    assert m(P(0x10000), 4, 16, 0, P(0x20000), s) == THETA
    assert m(P(0x10000), 4, 16, 128, P(0x20000), s) == THETA
    assert m(P(0x10000), -1, 16, 2, P(0x20000), s) == SHAPE
    assert m(P(0x10000), 4, (1 << 20) + 8, 2, P(0x20000), s) == SHAPE
    assert m(None, 4, 16, 2, P(0x20000), s) == NULL
    assert m(P(0x10000), 4, 16, 2, None, s) == NULL
    assert m(P(0x10000), 4, 16, 2, P(0x20002), s) == ALIGN
    # q occupies [0x10000, 0x10040); packed [0x10020, 0x10030) overlaps it
    assert m(P(0x10000), 4, 16, 2, P(0x10020), s) == ALIAS
    # nothing to do: valid without touching the device
    assert m(None, 0, 16, 2, None, s) == OK
    assert m(None, 4, 0, 2, None, s) == OK


def test_fwd_rejects(L):
    s = P(0)
    f = L.tern_linear_fwd
    X, pk, sc, Y = P(0x100000), P(0x200000), P(0x300000), P(0x400000)
    assert f(X, BF16, pk, sc, 64, 12, 64, Y, F32, s) == SHAPE      # in % 8
    assert f(X, BF16, pk, sc, 64, 64, 20, Y, F32, s) == SHAPE      # out % 8
    assert f(X, BF16, pk, sc, -1, 64, 64, Y, F32, s) == SHAPE
    assert f(X, 7, pk, sc, 64, 64, 64, Y, F32, s) == DTYPE
    assert f(X, F32, pk, sc, 64, 64, 64, Y, BF16, s) == DTYPE     # bf16 Y needs bf16 X
    assert f(None, BF16, pk, sc, 64, 64, 64, Y, F32, s) == NULL
    assert f(X, BF16, None, sc, 64, 64, 64, Y, F32, s) == NULL
    assert f(X, BF16, pk, None, 64, 64, 64, Y, F32, s) == NULL
    assert f(X, BF16, pk, sc, 64, 64, 64, None, F32, s) == NULL
    assert f(P(0x100008), BF16, pk, sc, 64, 64, 64, Y, F32, s) == ALIGN
    assert f(X, BF16, pk, P(0x300004), 64, 64, 64, Y, F32, s) == ALIGN
    assert f(X, BF16, P(0x200002), sc, 64, 64, 64, Y, F32, s) == ALIGN
    # Y [64, 64] fp32 = 16 KiB starting inside X [64, 64] bf16 = 8 KiB
    assert f(X, BF16, pk, sc, 64, 64, 64, P(0x101000), F32, s) == ALIAS
    assert f(X, BF16, pk, sc, 64, 64, 64, P(0x300000 - 0x100), F32, s) == ALIAS  # Y runs into scale
    # empty outputs: valid and nothing is enqueued
    assert f(None, BF16, pk, sc, 0, 64, 64, None, F32, s) == OK
    assert f(X, BF16, None, None, 64, 64, 0, None, F32, s) == OK


def test_bwd_rejects(L):
    s = P(0)
    b = L.tern_linear_bwd
    X, dY, pk, sc = P(0x1000000), P(0x2000000), P(0x3000000), P(0x4000000)
    dX, gq, sg = P(0x5000000), P(0x6000000), P(0x7000000)
    T, n_in, n_out = 4096, 2048, 2048
    need = tl.tern_linear_bwd_workspace_bytes(T, n_in, n_out)
    ws = P(0x10000000)
    assert b(X, dY, BF16, pk, sc, T, n_in, n_out, dX, BF16, gq, sg, ws, need, s) == DTYPE
    assert b(X, dY, 3, pk, sc, T, n_in, n_out, dX, F32, gq, sg, ws, need, s) == DTYPE
    assert b(X, dY, BF16, pk, sc, T, 100, n_out, dX, F32, gq, sg, ws, need, s) == SHAPE
    assert b(None, dY, BF16, pk, sc, T, n_in, n_out, dX, F32, gq, sg, ws, need, s) == NULL
    assert b(X, dY, BF16, pk, sc, T, n_in, n_out, dX, F32, None, sg, ws, need, s) == NULL
    assert b(X, dY, BF16, pk, sc, T, n_in, n_out, dX, F32, gq, None, ws, need, s) == NULL
    if need:
        assert b(X, dY, BF16, pk, sc, T, n_in, n_out, dX, F32, gq, sg, None, need, s) == WORKSPACE
        assert b(X, dY, BF16, pk, sc, T, n_in, n_out, dX, F32, gq, sg, ws, need - 1, s) == WORKSPACE
    assert b(X, dY, BF16, pk, sc, T, n_in, n_out, P(0x5000004), F32, gq, sg, ws, need, s) == ALIGN
    # gq [2048, 2048] fp32 = 16 MiB from 0x6000000 covers 0x7000000 (sgrad)
    assert b(X, dY, BF16, pk, sc, T, n_in, n_out, dX, F32, gq, sg, ws, need, s) == ALIAS
    # dX writes over dY
    assert b(X, dY, BF16, pk, sc, T, n_in, n_out, P(0x2000000 + 4096), F32, P(0x20000000), sg, ws, need,
             s) == ALIAS


def test_bwd_parts_reject(L):
    s = P(0)
    assert L.tern_linear_bwd_dx(P(0x1000), BF16, P(0x2000), P(0x3000), 8, 8, 8, P(0x4000), BF16, s) == DTYPE
    assert L.tern_linear_bwd_dx(None, BF16, P(0x2000), P(0x3000), 8, 8, 8, P(0x4000), F32, s) == NULL
    assert L.tern_linear_bwd_dw(P(0x1000), P(0x2000), BF16, P(0x3000), P(0x4000), 8, 8, 12, P(0x5000),
                                P(0x6000), P(0x7000), 1 << 20, s) == SHAPE


def test_workspace_bytes(L):
    """Three arguments, as the boundary states it: the workspace serves either
    activation type."""
    assert tl.SIGNATURES["tern_linear_bwd_workspace_bytes"][1] == [ctypes.c_int64] * 3
    assert tl.SIGNATURES["tern_linear_bwd_acc_workspace_bytes"][1] == [ctypes.c_int64] * 3
    assert tl.tern_linear_bwd_workspace_bytes(-1, 8, 8) == 0
    assert tl.tern_linear_bwd_workspace_bytes(8, 12, 8) == 0
    assert tl.tern_linear_bwd_workspace_bytes(0, 64, 64) == 0
    for (T, i, o) in [(64, 64, 64), (2048, 512, 512), (16384, 2048, 2048), (32768, 4096, 16384),
                      (1000, 200, 72), (4000, 1032, 1032)]:
        w = tl.tern_linear_bwd_workspace_bytes(T, i, o)
        # always room for at least one row of sgrad partials, 256-byte granular
        assert w >= 4 * o and w % 256 == 0, (T, i, o, w)
        assert tl.tern_linear_bwd_workspace_bytes(T, i, o) == w  # pure function


def test_bwd_accepts_the_three_argument_workspace(L):
    """A workspace of tern_linear_bwd_workspace_bytes(T, in, out) bytes passes
    the backward's workspace check for both activation types.  The checks run
    NULL, WORKSPACE, ALIGN, ALIAS in that order, so a misaligned dX reports
    ALIGN once the workspace is accepted, and one byte less reports
    WORKSPACE; nothing is launched either way."""
    s = P(0)
    b = L.tern_linear_bwd
    X, dY, pk, sc = P(0x1000000), P(0x2000000), P(0x3000000), P(0x4000000)
    gq, sg, ws, dX_bad = P(0x6000000), P(0x7000000), P(0x10000000), P(0x5000004)
    for (T, i, o) in [(4000, 1032, 1032), (16384, 2048, 2048), (2048, 512, 2048), (64, 64, 64)]:
        need = tl.tern_linear_bwd_workspace_bytes(T, i, o)
        assert need > 0
        for dt in (F32, BF16):
            assert b(X, dY, dt, pk, sc, T, i, o, dX_bad, F32, gq, sg, ws, need, s) == ALIGN, (T, i, o, dt)
        # at least one type needs every byte of it
        assert any(b(X, dY, dt, pk, sc, T, i, o, dX_bad, F32, gq, sg, ws, need - 1, s) == WORKSPACE
                   for dt in (F32, BF16)), (T, i, o)


def test_graph_calls_reject_missing_handles(L):
    """The graph calls refuse NULL streams and handles before any HIP call
    (NULL is the legacy default stream, which cannot record)."""
    h = ctypes.c_void_p(1234)
    assert L.tern_graph_begin(None) == NULL
    assert L.tern_graph_end(None, ctypes.byref(h)) == NULL
    assert h.value is None, "a failed tern_graph_end must leave a NULL handle"
    assert L.tern_graph_end(P(0x1000), None) == NULL
    assert L.tern_graph_launch(None, P(0x1000)) == NULL
    assert L.tern_graph_destroy(None) == OK


def test_acc_variants_reject(L):
    """The accumulating entry points apply the backward's checks; dW needs the
    larger accumulating workspace."""
    s = P(0)
    X, dY, pk, sc = P(0x1000000), P(0x2000000), P(0x3000000), P(0x4000000)
    dX, gq, sg = P(0x5000000), P(0x6000000), P(0x7000000)
    T, n_in, n_out = 4096, 2048, 2048
    dx = L.tern_linear_bwd_dx_acc
    assert dx(dY, 3, pk, sc, T, n_in, n_out, dX, s) == DTYPE
    assert dx(dY, BF16, pk, sc, T, 100, n_out, dX, s) == SHAPE
    assert dx(None, BF16, pk, sc, T, n_in, n_out, dX, s) == NULL
    assert dx(dY, BF16, pk, sc, T, n_in, n_out, None, s) == NULL
    assert dx(dY, BF16, pk, sc, T, n_in, n_out, P(0x5000004), s) == ALIGN
    assert dx(dY, BF16, pk, sc, T, n_in, n_out, P(0x2000000 + 4096), s) == ALIAS   # dX over dY
    dw = L.tern_linear_bwd_dw_acc
    need = tl.tern_linear_bwd_acc_workspace_bytes(T, n_in, n_out)
    plain = tl.tern_linear_bwd_workspace_bytes(T, n_in, n_out)
    assert need >= plain and need >= 4 * n_in * n_out   # room for G itself
    ws, gq2 = P(0x10000000), P(0x30000000)
    a = ctypes.c_float(0.5)
    assert dw(X, dY, BF16, pk, sc, T, n_in, n_out, a, gq2, sg, ws, need - 1, s) == WORKSPACE
    assert dw(X, dY, BF16, pk, sc, T, n_in, n_out, a, gq2, sg, None, need, s) == WORKSPACE
    assert dw(X, dY, BF16, pk, sc, T, n_in, 12, a, gq2, sg, ws, need, s) == SHAPE
    assert dw(None, dY, BF16, pk, sc, T, n_in, n_out, a, gq2, sg, ws, need, s) == NULL
    assert dw(X, dY, BF16, pk, sc, T, n_in, n_out, a, None, sg, ws, need, s) == NULL
    assert dw(X, dY, BF16, pk, sc, T, n_in, n_out, a, P(0x2000000 + 4096), sg, ws, need, s) == ALIAS  # gq over dY


def test_acc_workspace_bytes(L):
    assert tl.tern_linear_bwd_acc_workspace_bytes(8, 12, 8) == 0
    for (T, i, o) in [(64, 64, 64), (2048, 512, 2048), (16384, 8192, 2048), (1000, 200, 72)]:
        w = tl.tern_linear_bwd_acc_workspace_bytes(T, i, o)
        assert w >= tl.tern_linear_bwd_workspace_bytes(T, i, o) and w >= 4 * i * o and w % 256 == 0


def test_panel_rejects(L):
    s = P(0)
    assert L.tern_panel_reset(None, s) == NULL
    assert L.tern_panel_reset(P(0x1004), s) == ALIGN
    q, sc, pan = P(0x1000000), P(0x2000000), P(0x3000000)
    add = L.tern_panel_add
    assert add(q, -1, 64, 2, 7, None, sc, pan, s) == SHAPE
    assert add(q, 64, 64, 0, 7, None, sc, pan, s) == THETA
    assert add(q, 64, 64, 2, 129, None, sc, pan, s) == THETA
    assert add(None, 64, 64, 2, 7, None, sc, pan, s) == NULL
    assert add(q, 64, 64, 2, 7, None, None, pan, s) == NULL
    assert add(q, 64, 64, 2, 7, None, sc, None, s) == NULL
    assert add(q, 64, 64, 2, 7, None, sc, P(0x3000004), s) == ALIGN
    assert add(q, 64, 64, 2, 7, P(0x4000002), sc, pan, s) == ALIGN
    assert add(q, 64, 64, 2, 7, None, sc, P(0x1000000 + 64), s) == ALIAS   # panel inside q


def test_group_gather_rejects(L):
    s = P(0)
    g = L.tern_group_gather
    q = (ctypes.c_void_p * 2)(0x1000000, 0x2000000)
    sc = (ctypes.c_void_p * 2)(0x3000000, 0x3100000)
    outs = (ctypes.c_int64 * 2)(64, 128)
    qg, sg = P(0x4000000), P(0x5000000)
    assert g(q, sc, outs, 0, 64, qg, sg, s) == SHAPE
    assert g(q, sc, outs, 9, 64, qg, sg, s) == SHAPE
    assert g(q, sc, outs, 2, -1, qg, sg, s) == SHAPE
    assert g(q, sc, (ctypes.c_int64 * 2)(64, -8), 2, 64, qg, sg, s) == SHAPE
    assert g(None, sc, outs, 2, 64, qg, sg, s) == NULL
    assert g(q, sc, outs, 2, 64, None, sg, s) == NULL
    assert g((ctypes.c_void_p * 2)(0x1000000, None), sc, outs, 2, 64, qg, sg, s) == NULL
    assert g(q, sc, outs, 2, 64, P(0x1000000 + 100), sg, s) == ALIAS      # q_group over member 0's q
    assert g(q, sc, outs, 2, 64, qg, P(0x4000000 + 64), s) == ALIAS       # scale_group inside q_group


def test_scale_adamw_rejects(L):
    s = P(0)
    f = L.tern_scale_adamw
    sg, sc, m, v = P(0x1000000), P(0x2000000), P(0x3000000), P(0x4000000)
    hp = [ctypes.c_float(x) for x in (1e-3, 1e-3, 0.9, 0.999, 1e-8, 0.0)]
    VALUE = -9
    assert f(sg, sc, m, v, -1, 1, *hp, s) == SHAPE
    assert f(sg, sc, m, v, 64, 0, *hp, s) == VALUE
    assert f(sg, sc, m, v, 64, 1, ctypes.c_float(0.0), *hp[1:], s) == VALUE
    assert f(sg, sc, m, v, 64, 1, hp[0], ctypes.c_float(float("inf")), *hp[2:], s) == VALUE
    assert f(None, sc, m, v, 64, 1, *hp, s) == NULL
    assert f(sg, sc, None, v, 64, 1, *hp, s) == NULL
    assert f(sg, P(0x2000002), m, v, 64, 1, *hp, s) == ALIGN
    assert f(sg, sc, P(0x2000000 + 128), v, 64, 1, *hp, s) == ALIAS   # m overlaps scale
    assert f(sg, sc, m, v, 0, 1, *hp, s) == OK                       # nothing to update


def test_noalloc_rejects_before_any_hip_call(L):
    """The allocation-free backward applies tern_linear_bwd's checks before it
    looks up its scratch (no GPU here: any HIP call would fail with HIP)."""
    s = P(0)
    f = L.tern_linear_bwd_noalloc
    X, dY, pk, sc = P(0x1000000), P(0x2000000), P(0x3000000), P(0x4000000)
    dX, gq, sg = P(0x5000000), P(0x6000000), P(0x7000000)
    T, n_in, n_out = 4096, 1024, 1024
    assert f(X, dY, BF16, pk, sc, T, n_in, n_out, dX, BF16, gq, sg, s) == DTYPE
    assert f(X, dY, 3, pk, sc, T, n_in, n_out, dX, F32, gq, sg, s) == DTYPE
    assert f(X, dY, BF16, pk, sc, T, 100, n_out, dX, F32, gq, sg, s) == SHAPE
    assert f(None, dY, BF16, pk, sc, T, n_in, n_out, dX, F32, gq, sg, s) == NULL
    assert f(X, dY, BF16, pk, sc, T, n_in, n_out, dX, F32, None, sg, s) == NULL
    assert f(X, dY, BF16, pk, sc, T, n_in, n_out, P(0x5000004), F32, gq, sg, s) == ALIGN
    assert f(X, dY, BF16, pk, sc, T, n_in, n_out, P(0x2000000 + 4096), F32, P(0x20000000), sg, s) == ALIAS
    # the largest in * out with an sgrad partial table above 64 MiB
    big = [P(k << 40) for k in range(1, 8)]   # far apart: no overlap at these sizes
    assert f(big[0], big[1], BF16, big[2], big[3], 64, 1 << 20, 1 << 14, big[4], F32, big[5], big[6], s) == -10


def _projs(n, shapes, base=1 << 40):
    """tern_proj_t array with every pointer in its own 1 GiB window."""
    arr = (tl.TernProj * n)()
    for i, (ni, no) in enumerate(shapes):
        arr[i].in_, arr[i].out = ni, no
        for j, f in enumerate(("q", "tern_packed", "scale", "X", "dY", "Y", "dX", "gq", "sgrad")):
            setattr(arr[i], f, base + ((i * 16 + j) << 30))
    return arr


def test_layer_calls_reject(L):
    """The layer calls check every projection and the aliasing across them
    before any HIP call."""
    s = P(0)
    shapes = [(512, 512), (512, 2048), (2048, 512)]
    a = _projs(3, shapes)
    T = 2048
    assert L.tern_layer_fwd(a, 0, T, BF16, F32, s) == SHAPE
    assert L.tern_layer_fwd(a, 9, T, BF16, F32, s) == SHAPE
    assert L.tern_layer_fwd(None, 3, T, BF16, F32, s) == NULL
    assert L.tern_layer_fwd(a, 3, T, 5, F32, s) == DTYPE
    assert L.tern_layer_fwd(a, 3, T, F32, BF16, s) == DTYPE
    b = _projs(3, shapes)
    b[1].out = 2044
    assert L.tern_layer_fwd(b, 3, T, BF16, F32, s) == SHAPE
    b = _projs(3, shapes)
    b[2].X = None
    assert L.tern_layer_fwd(b, 3, T, BF16, F32, s) == NULL
    b = _projs(3, shapes)
    b[2].Y = b[2].Y + 4
    assert L.tern_layer_fwd(b, 3, T, BF16, F32, s) == ALIGN
    b = _projs(3, shapes)
    b[2].Y = b[0].X          # projection 2 writes over projection 0's input
    assert L.tern_layer_fwd(b, 3, T, BF16, F32, s) == ALIAS
    b = _projs(3, shapes)
    b[1].Y = b[0].Y + 256    # two outputs overlap
    assert L.tern_layer_fwd(b, 3, T, BF16, F32, s) == ALIAS
    b = _projs(3, shapes)
    b[1].X = b[0].X          # a shared input is fine: stops at the (absent) device, not at ALIAS
    b[1].dX = b[1].dX + 4
    assert L.tern_layer_bwd_dx(b, 3, T, BF16, s) == ALIGN
    b = _projs(3, shapes)
    b[0].dX = b[2].dY
    assert L.tern_layer_bwd_dx(b, 3, T, BF16, s) == ALIAS
    # dW: workspace size and overlap
    need = L.tern_layer_bwd_dw_workspace_bytes(a, 3, T)
    assert need > 0 and need % 256 == 0
    ws = P(1 << 44)
    assert L.tern_layer_bwd_dw(a, 3, T, BF16, None, need, s) == WORKSPACE
    assert L.tern_layer_bwd_dw(a, 3, T, BF16, ws, need - 1, s) == WORKSPACE
    assert L.tern_layer_bwd_dw(a, 3, T, BF16, P(a[0].X), need, s) == ALIAS   # workspace over an input
    b = _projs(3, shapes)
    b[1].sgrad = None
    assert L.tern_layer_bwd_dw(b, 3, T, BF16, ws, need, s) == NULL
    # materialize: theta, shared handles
    assert L.tern_layer_materialize(a, 3, 0, s) == THETA
    b = _projs(3, shapes)
    b[1].tern_packed = b[0].tern_packed
    assert L.tern_layer_materialize(b, 3, 2, s) == ALIAS
    assert L.tern_layer_bwd_dw_workspace_bytes(a, 0, T) == 0


def test_layer_workspace_covers_either_type(L):
    """The layer workspace covers the grouped plan (bf16) and the per-projection
    plans (fp32), and is at least the sum of the sgrad partial tables."""
    for T, shapes in ((2048, [(512, 512)] * 4 + [(512, 2048), (2048, 512)]),
                      (16384, [(2048, 2048)] * 4 + [(2048, 8192), (8192, 2048)]),
                      (1000, [(64, 1024), (1024, 40), (256, 256)])):
        a = _projs(len(shapes), shapes)
        need = L.tern_layer_bwd_dw_workspace_bytes(a, len(shapes), T)
        single = sum(tl.tern_linear_bwd_workspace_bytes(T, i, o) for i, o in shapes)
        assert need >= min(single, sum(4 * o for _, o in shapes)), (T, need, single)
        assert tl.tern_layer_bwd_dw_workspace_bytes(shapes, T) == need

