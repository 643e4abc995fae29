"""Python binding of libtern, the MI355X forward and backward of the SR4
ternary projection (C ABI in include/tern.h).

The functions below carry the C entry points' names and only marshal
arguments: torch tensors (device memory) become raw pointers, the current HIP
stream becomes the stream handle, and a nonzero status becomes a ``TernError``.
Every computation runs in the HIP kernels of libtern.so; there is no fallback.
If the library has not been built, the first call raises.

Build it in-tree with ``python -m ternary_weight_linear_tern_amd.build``.
"""
from __future__ import annotations

import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libtern.so")

TERN_F32 = 0
TERN_BF16 = 1

STATUS = {
    0: "TERN_OK", -1: "TERN_ERR_NULL", -2: "TERN_ERR_SHAPE", -3: "TERN_ERR_THETA",
    -4: "TERN_ERR_DTYPE", -5: "TERN_ERR_ALIGN", -6: "TERN_ERR_WORKSPACE", -7: "TERN_ERR_ALIAS",
    -8: "TERN_ERR_HIP", -9: "TERN_ERR_VALUE",
}

# Every symbol include/tern.h declares: name -> (restype, argtypes)
_vp, _i64, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
SIGNATURES = {
    "tern_packed_words": (_i64, [_i64, _i64]),
    "tern_materialize": (ctypes.c_int, [_vp, _i64, _i64, _i32, _vp, _vp]),
    "tern_linear_fwd": (ctypes.c_int, [_vp, _i32, _vp, _vp, _i64, _i64, _i64, _vp, _i32, _vp]),
    "tern_linear_bwd_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32]),
    "tern_linear_bwd": (ctypes.c_int, [_vp, _vp, _i32, _vp, _vp, _i64, _i64, _i64, _vp, _i32, _vp,
                                       _vp, _vp, _sz, _vp]),
    "tern_linear_bwd_dx": (ctypes.c_int, [_vp, _i32, _vp, _vp, _i64, _i64, _i64, _vp, _i32, _vp]),
    "tern_linear_bwd_dw": (ctypes.c_int, [_vp, _vp, _i32, _vp, _vp, _i64, _i64, _i64, _vp, _vp,
                                          _vp, _sz, _vp]),
    "tern_linear_bwd_dx_acc": (ctypes.c_int, [_vp, _i32, _vp, _vp, _i64, _i64, _i64, _vp, _vp]),
    "tern_linear_bwd_acc_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32]),
    "tern_linear_bwd_dw_acc": (ctypes.c_int, [_vp, _vp, _i32, _vp, _vp, _i64, _i64, _i64, ctypes.c_float,
                                              _vp, _vp, _vp, _sz, _vp]),
    "tern_group_gather": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i64, _vp, _vp, _vp]),
    "tern_scale_adamw": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i32] + [ctypes.c_float] * 6 + [_vp]),
    "tern_panel_reset": (ctypes.c_int, [_vp, _vp]),
    "tern_panel_add": (ctypes.c_int, [_vp, _i64, _i64, _i32, _i32, _vp, _vp, _vp, _vp]),
    "tern_graph_begin": (ctypes.c_int, [_vp]),
    "tern_graph_end": (ctypes.c_int, [_vp, ctypes.POINTER(_vp)]),
    "tern_graph_launch": (ctypes.c_int, [_vp, _vp]),
    "tern_graph_destroy": (ctypes.c_int, [_vp]),
    "tern_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "tern_version": (ctypes.c_char_p, []),
}


class TernError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({tern_status_str(status)})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libtern.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m ternary_weight_linear_tern_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libtern must be contiguous")
    return ctypes.c_void_p(t.data_ptr()) if t.numel() else None


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _act_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return TERN_BF16
    if t.dtype == torch.float32:
        return TERN_F32
    raise TypeError(f"activation dtype must be bfloat16 or float32, got {t.dtype}")


def _check(fn: str, rc: int):
    if rc != 0:
        raise TernError(fn, rc)


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def tern_status_str(status: int) -> str:
    return lib().tern_status_str(int(status)).decode()


def tern_version() -> str:
    return lib().tern_version().decode()


def tern_packed_words(n_in: int, n_out: int) -> int:
    return int(lib().tern_packed_words(n_in, n_out))


def tern_linear_bwd_workspace_bytes(T: int, n_in: int, n_out: int, act_dtype) -> int:
    code = act_dtype if isinstance(act_dtype, int) else (
        TERN_BF16 if act_dtype == torch.bfloat16 else TERN_F32)
    return int(lib().tern_linear_bwd_workspace_bytes(T, n_in, n_out, code))


def tern_materialize(q: torch.Tensor, theta: int, tern_packed: torch.Tensor, stream=None) -> None:
    """q int8 [in, out] -> packed ternary handle (see empty_packed)."""
    n_in, n_out = q.shape
    rc = lib().tern_materialize(_ptr(q), n_in, n_out, int(theta), _ptr(tern_packed), _stream(stream))
    _check("tern_materialize", rc)


def tern_linear_fwd(X: torch.Tensor, tern_packed: torch.Tensor, scale: torch.Tensor, Y: torch.Tensor,
                    stream=None) -> None:
    """Y [T, out] (fp32 or bf16) = X [T, in] . (scale * tern)."""
    T, n_in = X.shape
    n_out = scale.shape[0]
    rc = lib().tern_linear_fwd(_ptr(X), _act_code(X), _ptr(tern_packed), _ptr(scale), T, n_in, n_out,
                               _ptr(Y), _act_code(Y), _stream(stream))
    _check("tern_linear_fwd", rc)


def tern_linear_bwd(X, dY, tern_packed, scale, dX, gq, sgrad, workspace, stream=None) -> None:
    T, n_in = X.shape
    n_out = scale.shape[0]
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().tern_linear_bwd(_ptr(X), _ptr(dY), _act_code(X), _ptr(tern_packed), _ptr(scale), T,
                               n_in, n_out, _ptr(dX), _act_code(dX), _ptr(gq), _ptr(sgrad),
                               _ptr(workspace), ws_bytes, _stream(stream))
    _check("tern_linear_bwd", rc)


def tern_linear_bwd_dx(dY, tern_packed, scale, dX, n_in: int | None = None, stream=None) -> None:
    T, n_out = dY.shape
    n_in = dX.shape[1] if n_in is None else n_in
    rc = lib().tern_linear_bwd_dx(_ptr(dY), _act_code(dY), _ptr(tern_packed), _ptr(scale), T, n_in,
                                  n_out, _ptr(dX), _act_code(dX), _stream(stream))
    _check("tern_linear_bwd_dx", rc)


def tern_linear_bwd_dw(X, dY, tern_packed, scale, gq, sgrad, workspace, stream=None) -> None:
    T, n_in = X.shape
    n_out = scale.shape[0]
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().tern_linear_bwd_dw(_ptr(X), _ptr(dY), _act_code(X), _ptr(tern_packed), _ptr(scale), T,
                                  n_in, n_out, _ptr(gq), _ptr(sgrad), _ptr(workspace), ws_bytes,
                                  _stream(stream))
    _check("tern_linear_bwd_dw", rc)


def tern_linear_bwd_dx_acc(dY, tern_packed, scale, dX, n_in: int | None = None, stream=None) -> None:
    """dX (fp32) += dY . (scale * tern)^T."""
    T, n_out = dY.shape
    n_in = dX.shape[1] if n_in is None else n_in
    if dX.dtype != torch.float32:
        raise TypeError("dX must be float32")
    rc = lib().tern_linear_bwd_dx_acc(_ptr(dY), _act_code(dY), _ptr(tern_packed), _ptr(scale), T, n_in, n_out,
                                      _ptr(dX), _stream(stream))
    _check("tern_linear_bwd_dx_acc", rc)


def tern_linear_bwd_acc_workspace_bytes(T: int, n_in: int, n_out: int, act_dtype) -> int:
    code = act_dtype if isinstance(act_dtype, int) else (
        TERN_BF16 if act_dtype == torch.bfloat16 else TERN_F32)
    return int(lib().tern_linear_bwd_acc_workspace_bytes(T, n_in, n_out, code))


def tern_linear_bwd_dw_acc(X, dY, tern_packed, scale, gq, sgrad, workspace, alpha: float = 1.0,
                           stream=None) -> None:
    """gq += alpha * G * scale, sgrad += alpha * sum_r G * tern (G = X^T . dY)."""
    T, n_in = X.shape
    n_out = scale.shape[0]
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().tern_linear_bwd_dw_acc(_ptr(X), _ptr(dY), _act_code(X), _ptr(tern_packed), _ptr(scale), T,
                                      n_in, n_out, float(alpha), _ptr(gq), _ptr(sgrad), _ptr(workspace),
                                      ws_bytes, _stream(stream))
    _check("tern_linear_bwd_dw_acc", rc)


def tern_group_gather(qs, scales, q_group: torch.Tensor, scale_group: torch.Tensor, stream=None) -> None:
    """q_group [in, sum out] and scale_group [sum out] from the members' q
    [in, out_i] and scale [out_i] (projections that read one input)."""
    n = len(qs)
    n_in = qs[0].shape[0] if n else 0
    qa = (_vp * max(n, 1))(*[_ptr(t) for t in qs])
    sa = (_vp * max(n, 1))(*[_ptr(t) for t in scales])
    oa = (_i64 * max(n, 1))(*[int(t.shape[1]) for t in qs])
    rc = lib().tern_group_gather(qa, sa, oa, n, n_in, _ptr(q_group), _ptr(scale_group), _stream(stream))
    _check("tern_group_gather", rc)


def tern_scale_adamw(sgrad, scale, m, v, step: int, lr: float, scale_lr: float | None = None, b1: float = 0.9,
                     b2: float = 0.999, eps: float = 1e-8, wd: float = 0.0, stream=None) -> None:
    """AdamW step of the per-column scale from its gradient (in place on
    scale, m, v; scale_lr defaults to lr)."""
    sl = lr if scale_lr is None else scale_lr
    rc = lib().tern_scale_adamw(_ptr(sgrad), _ptr(scale), _ptr(m), _ptr(v), int(scale.shape[0]), int(step),
                                float(lr), float(sl), float(b1), float(b2), float(eps), float(wd),
                                _stream(stream))
    _check("tern_scale_adamw", rc)


PANEL_COUNTS = ("total", "neg", "zero", "pos", "rail", "dead", "churn", "churn_total", "scale_count")
PANEL_STATS = ("scale_sum", "scale_min", "scale_max")


def empty_panel(device="cuda") -> torch.Tensor:
    """Device storage of one tern_panel_t (9 uint64 counts, then 3 doubles)."""
    return torch.empty((len(PANEL_COUNTS) + len(PANEL_STATS),), dtype=torch.float64, device=device)


def tern_panel_reset(panel: torch.Tensor, stream=None) -> None:
    _check("tern_panel_reset", lib().tern_panel_reset(_ptr(panel), _stream(stream)))


def tern_panel_add(q: torch.Tensor, theta: int, scale: torch.Tensor, panel: torch.Tensor, prev_packed=None,
                   q_clamp: int = 7, stream=None) -> None:
    """Add one ternary matrix (q int8 [in, out], scale [out]) to the panel;
    prev_packed: the previous step's handle for churn, or None."""
    n_in, n_out = q.shape
    rc = lib().tern_panel_add(_ptr(q), n_in, n_out, int(theta), int(q_clamp), _ptr(prev_packed), _ptr(scale),
                              _ptr(panel), _stream(stream))
    _check("tern_panel_add", rc)


def panel_values(panel: torch.Tensor) -> dict:
    """The accumulator's fields, and the page's fractions of them (churn only
    when every element was compared with a previous handle)."""
    h = panel.cpu()
    n = len(PANEL_COUNTS)
    counts = h[:n].view(torch.int64).tolist()
    r = dict(zip(PANEL_COUNTS, counts))
    r.update(zip(PANEL_STATS, h[n:].tolist()))
    dt = float(r["total"]) if r["total"] else 1.0
    valid = r["total"] > 0 and r["churn_total"] == r["total"]
    r.update(pct_neg=r["neg"] / dt, pct_zero=r["zero"] / dt, pct_pos=r["pos"] / dt, rail_pct=r["rail"] / dt,
             dead_pct=r["dead"] / dt, churn_frac=r["churn"] / dt if valid else 0.0,
             scale_mean=r["scale_sum"] / r["scale_count"] if r["scale_count"] else 0.0)
    return r


def tern_graph_begin(stream) -> None:
    """Start recording the library calls enqueued on `stream` (a created
    torch.cuda.Stream or raw handle, not the legacy default stream)."""
    _check("tern_graph_begin", lib().tern_graph_begin(_stream(stream)))


def tern_graph_end(stream) -> ctypes.c_void_p:
    """Stop recording on `stream`; returns the instantiated graph's handle
    (release it with tern_graph_destroy)."""
    h = _vp()
    _check("tern_graph_end", lib().tern_graph_end(_stream(stream), ctypes.byref(h)))
    return h


def tern_graph_launch(graph, stream=None) -> None:
    _check("tern_graph_launch", lib().tern_graph_launch(graph, _stream(stream)))


def tern_graph_destroy(graph) -> None:
    _check("tern_graph_destroy", lib().tern_graph_destroy(graph))


# ---------------------------------------------------------------------------
# allocation helpers (torch owns the memory; the library never allocates)
# ---------------------------------------------------------------------------

def empty_packed(n_in: int, n_out: int, device="cuda") -> torch.Tensor:
    """A packed ternary handle: tern_packed_words(n_in, n_out) int32 words."""
    return torch.empty((max(tern_packed_words(n_in, n_out), 1),), dtype=torch.int32, device=device)


def packed_canonical(tern_packed: torch.Tensor, n_in: int, n_out: int) -> torch.Tensor:
    """View of the canonical 2-bit matrix at the start of a packed handle:
    [n_in, ceil(n_out / 16)] words, code of (r, c) at bits 2 (c % 16) of word
    (r, c / 16)."""
    wpr = (n_out + 15) // 16
    return tern_packed.reshape(-1)[: n_in * wpr].view(n_in, wpr)


def empty_workspace(T: int, n_in: int, n_out: int, act_dtype, device="cuda", acc: bool = False) -> torch.Tensor:
    """Workspace of tern_linear_bwd / tern_linear_bwd_dw (acc: of tern_linear_bwd_dw_acc)."""
    q = tern_linear_bwd_acc_workspace_bytes if acc else tern_linear_bwd_workspace_bytes
    nbytes = q(T, n_in, n_out, act_dtype)
    return torch.empty((max(nbytes, 16) // 16, 16), dtype=torch.uint8, device=device)
