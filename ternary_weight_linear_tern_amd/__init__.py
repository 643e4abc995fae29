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
    -8: "TERN_ERR_HIP", -9: "TERN_ERR_VALUE", -10: "TERN_ERR_SCRATCH",
}

# Every symbol include/tern.h declares: name -> (restype, argtypes)
_vp, _i64, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
SIGNATURES = {
    "tern_packed_words": (_i64, [_i64, _i64]),
    "tern_materialize": (ctypes.c_int, [_vp, _i64, _i64, _i32, _vp, _vp]),
    "tern_linear_fwd": (ctypes.c_int, [_vp, _i32, _vp, _vp, _i64, _i64, _i64, _vp, _i32, _vp]),
    "tern_linear_bwd_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "tern_linear_bwd": (ctypes.c_int, [_vp, _vp, _i32, _vp, _vp, _i64, _i64, _i64, _vp, _i32, _vp,
                                       _vp, _vp, _sz, _vp]),
    "tern_linear_bwd_noalloc": (ctypes.c_int, [_vp, _vp, _i32, _vp, _vp, _i64, _i64, _i64, _vp, _i32, _vp,
                                               _vp, _vp]),
    "tern_linear_bwd_dx": (ctypes.c_int, [_vp, _i32, _vp, _vp, _i64, _i64, _i64, _vp, _i32, _vp]),
    "tern_linear_bwd_dw": (ctypes.c_int, [_vp, _vp, _i32, _vp, _vp, _i64, _i64, _i64, _vp, _vp,
                                          _vp, _sz, _vp]),
    "tern_linear_bwd_dx_acc": (ctypes.c_int, [_vp, _i32, _vp, _vp, _i64, _i64, _i64, _vp, _vp]),
    "tern_linear_bwd_acc_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "tern_linear_bwd_dw_acc": (ctypes.c_int, [_vp, _vp, _i32, _vp, _vp, _i64, _i64, _i64, ctypes.c_float,
                                              _vp, _vp, _vp, _sz, _vp]),
    "tern_group_gather": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i64, _vp, _vp, _vp]),
    "tern_scale_adamw": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i32] + [ctypes.c_float] * 6 + [_vp]),
    "tern_panel_reset": (ctypes.c_int, [_vp, _vp]),
    "tern_panel_add": (ctypes.c_int, [_vp, _i64, _i64, _i32, _i32, _vp, _vp, _vp, _vp]),
    "tern_panel_fractions": (ctypes.c_int, [_vp, _vp]),
    "tern_layer_materialize": (ctypes.c_int, [_vp, _i32, _i32, _vp]),
    "tern_layer_fwd": (ctypes.c_int, [_vp, _i32, _i64, _i32, _i32, _vp]),
    "tern_layer_bwd_dx": (ctypes.c_int, [_vp, _i32, _i64, _i32, _vp]),
    "tern_layer_bwd_dw_workspace_bytes": (_sz, [_vp, _i32, _i64]),
    "tern_layer_bwd_dw": (ctypes.c_int, [_vp, _i32, _i64, _i32, _vp, _sz, _vp]),
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


_F32 = (torch.float32,)
_ACT = (torch.bfloat16, torch.float32)


def _need(fn: str, name: str, t, shape, dtypes) -> None:
    """t must be a tensor of this shape and one of these dtypes."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{fn}: {name} must be a tensor")
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{fn}: {name} has shape {tuple(t.shape)}, expected {tuple(int(x) for x in shape)}")
    if t.dtype not in dtypes:
        raise TypeError(f"{fn}: {name} has dtype {t.dtype}, expected one of {dtypes}")


def _need_bytes(fn: str, name: str, t, nbytes: int) -> None:
    """t must hold at least nbytes (a packed handle, a workspace, a panel)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{fn}: {name} must be a tensor")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{fn}: {name} holds {have} bytes, needs {nbytes}")


def _need_packed(fn: str, t, n_in: int, n_out: int) -> None:
    if not isinstance(t, torch.Tensor) or t.dtype not in (torch.int32, torch.uint32):
        raise TypeError(f"{fn}: tern_packed must be an int32 tensor (see empty_packed)")
    _need_bytes(fn, "tern_packed", t, 4 * max(tern_packed_words(n_in, n_out), 0))


def _need_device(fn: str, *ts) -> None:
    """Every tensor passed to the library lives on one GPU."""
    devs = {t.device for t in ts if isinstance(t, torch.Tensor)}
    if any(d.type != "cuda" for d in devs):
        raise ValueError(f"{fn}: every tensor must be on a GPU (got {sorted(map(str, devs))})")
    if len(devs) > 1:
        raise ValueError(f"{fn}: tensors on several devices {sorted(map(str, devs))}")


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def tern_status_str(status: int) -> str:
    return lib().tern_status_str(int(status)).decode()


def tern_version() -> str:
    return lib().tern_version().decode()


def tern_packed_words(n_in: int, n_out: int) -> int:
    return int(lib().tern_packed_words(n_in, n_out))


def tern_linear_bwd_workspace_bytes(T: int, n_in: int, n_out: int) -> int:
    return int(lib().tern_linear_bwd_workspace_bytes(T, n_in, n_out))


def tern_materialize(q: torch.Tensor, theta: int, tern_packed: torch.Tensor, stream=None) -> None:
    """q int8 [in, out] -> packed ternary handle (see empty_packed)."""
    fn = "tern_materialize"
    if q.dim() != 2:
        raise ValueError(f"{fn}: q must be [in, out]")
    n_in, n_out = q.shape
    _need(fn, "q", q, (n_in, n_out), (torch.int8,))
    _need_packed(fn, tern_packed, n_in, n_out)
    _need_device(fn, q, tern_packed)
    rc = lib().tern_materialize(_ptr(q), n_in, n_out, int(theta), _ptr(tern_packed), _stream(stream))
    _check("tern_materialize", rc)


def tern_linear_fwd(X: torch.Tensor, tern_packed: torch.Tensor, scale: torch.Tensor, Y: torch.Tensor,
                    stream=None) -> None:
    """Y [T, out] (fp32 or bf16) = X [T, in] . (scale * tern)."""
    fn = "tern_linear_fwd"
    if X.dim() != 2 or scale.dim() != 1:
        raise ValueError(f"{fn}: X must be [T, in] and scale [out]")
    T, n_in = X.shape
    n_out = scale.shape[0]
    _need(fn, "X", X, (T, n_in), _ACT)
    _need(fn, "scale", scale, (n_out,), _F32)
    _need(fn, "Y", Y, (T, n_out), (torch.float32, X.dtype))
    _need_packed(fn, tern_packed, n_in, n_out)
    _need_device(fn, X, tern_packed, scale, Y)
    rc = lib().tern_linear_fwd(_ptr(X), _act_code(X), _ptr(tern_packed), _ptr(scale), T, n_in, n_out,
                               _ptr(Y), _act_code(Y), _stream(stream))
    _check("tern_linear_fwd", rc)


def _bwd_dw_checks(fn, X, dY, tern_packed, scale, gq, sgrad, workspace):
    if X.dim() != 2 or scale.dim() != 1:
        raise ValueError(f"{fn}: X must be [T, in] and scale [out]")
    T, n_in = X.shape
    n_out = scale.shape[0]
    _need(fn, "X", X, (T, n_in), _ACT)
    _need(fn, "dY", dY, (T, n_out), (X.dtype,))
    _need(fn, "scale", scale, (n_out,), _F32)
    _need(fn, "gq", gq, (n_in, n_out), _F32)
    _need(fn, "sgrad", sgrad, (n_out,), _F32)
    _need_packed(fn, tern_packed, n_in, n_out)
    if workspace is not None:
        _need_bytes(fn, "workspace", workspace, 0)
    return T, n_in, n_out


def tern_linear_bwd(X, dY, tern_packed, scale, dX, gq, sgrad, workspace, stream=None) -> None:
    fn = "tern_linear_bwd"
    T, n_in, n_out = _bwd_dw_checks(fn, X, dY, tern_packed, scale, gq, sgrad, workspace)
    _need(fn, "dX", dX, (T, n_in), _F32)
    _need_device(fn, X, dY, tern_packed, scale, dX, gq, sgrad, workspace)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().tern_linear_bwd(_ptr(X), _ptr(dY), _act_code(X), _ptr(tern_packed), _ptr(scale), T,
                               n_in, n_out, _ptr(dX), _act_code(dX), _ptr(gq), _ptr(sgrad),
                               _ptr(workspace), ws_bytes, _stream(stream))
    _check("tern_linear_bwd", rc)


def tern_linear_bwd_noalloc(X, dY, tern_packed, scale, dX, gq, sgrad, stream=None) -> None:
    """tern_linear_bwd without a workspace: the library's static scratch is
    used (calls that overlap on one GPU race)."""
    fn = "tern_linear_bwd_noalloc"
    T, n_in, n_out = _bwd_dw_checks(fn, X, dY, tern_packed, scale, gq, sgrad, None)
    _need(fn, "dX", dX, (T, n_in), _F32)
    _need_device(fn, X, dY, tern_packed, scale, dX, gq, sgrad)
    rc = lib().tern_linear_bwd_noalloc(_ptr(X), _ptr(dY), _act_code(X), _ptr(tern_packed), _ptr(scale), T,
                                       n_in, n_out, _ptr(dX), _act_code(dX), _ptr(gq), _ptr(sgrad),
                                       _stream(stream))
    _check(fn, rc)


def _bwd_dx_checks(fn, dY, tern_packed, scale, dX, n_in):
    if dY.dim() != 2 or scale.dim() != 1 or dX.dim() != 2:
        raise ValueError(f"{fn}: dY must be [T, out], scale [out] and dX [T, in]")
    T, n_out = dY.shape
    n_in = dX.shape[1] if n_in is None else n_in
    _need(fn, "dY", dY, (T, n_out), _ACT)
    _need(fn, "scale", scale, (n_out,), _F32)
    _need(fn, "dX", dX, (T, n_in), _F32)
    _need_packed(fn, tern_packed, n_in, n_out)
    _need_device(fn, dY, tern_packed, scale, dX)
    return T, n_in, n_out


def tern_linear_bwd_dx(dY, tern_packed, scale, dX, n_in: int | None = None, stream=None) -> None:
    T, n_in, n_out = _bwd_dx_checks("tern_linear_bwd_dx", dY, tern_packed, scale, dX, n_in)
    rc = lib().tern_linear_bwd_dx(_ptr(dY), _act_code(dY), _ptr(tern_packed), _ptr(scale), T, n_in,
                                  n_out, _ptr(dX), _act_code(dX), _stream(stream))
    _check("tern_linear_bwd_dx", rc)


def tern_linear_bwd_dw(X, dY, tern_packed, scale, gq, sgrad, workspace, stream=None) -> None:
    fn = "tern_linear_bwd_dw"
    T, n_in, n_out = _bwd_dw_checks(fn, X, dY, tern_packed, scale, gq, sgrad, workspace)
    _need_device(fn, X, dY, tern_packed, scale, gq, sgrad, workspace)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().tern_linear_bwd_dw(_ptr(X), _ptr(dY), _act_code(X), _ptr(tern_packed), _ptr(scale), T,
                                  n_in, n_out, _ptr(gq), _ptr(sgrad), _ptr(workspace), ws_bytes,
                                  _stream(stream))
    _check("tern_linear_bwd_dw", rc)


def tern_linear_bwd_dx_acc(dY, tern_packed, scale, dX, n_in: int | None = None, stream=None) -> None:
    """dX (fp32) += dY . (scale * tern)^T."""
    T, n_in, n_out = _bwd_dx_checks("tern_linear_bwd_dx_acc", dY, tern_packed, scale, dX, n_in)
    rc = lib().tern_linear_bwd_dx_acc(_ptr(dY), _act_code(dY), _ptr(tern_packed), _ptr(scale), T, n_in, n_out,
                                      _ptr(dX), _stream(stream))
    _check("tern_linear_bwd_dx_acc", rc)


def tern_linear_bwd_acc_workspace_bytes(T: int, n_in: int, n_out: int) -> int:
    return int(lib().tern_linear_bwd_acc_workspace_bytes(T, n_in, n_out))


def tern_linear_bwd_dw_acc(X, dY, tern_packed, scale, gq, sgrad, workspace, alpha: float = 1.0,
                           stream=None) -> None:
    """gq += alpha * G * scale, sgrad += alpha * sum_r G * tern (G = X^T . dY)."""
    fn = "tern_linear_bwd_dw_acc"
    T, n_in, n_out = _bwd_dw_checks(fn, X, dY, tern_packed, scale, gq, sgrad, workspace)
    _need_device(fn, X, dY, tern_packed, scale, gq, sgrad, workspace)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().tern_linear_bwd_dw_acc(_ptr(X), _ptr(dY), _act_code(X), _ptr(tern_packed), _ptr(scale), T,
                                      n_in, n_out, float(alpha), _ptr(gq), _ptr(sgrad), _ptr(workspace),
                                      ws_bytes, _stream(stream))
    _check("tern_linear_bwd_dw_acc", rc)


def tern_group_gather(qs, scales, q_group: torch.Tensor, scale_group: torch.Tensor, stream=None) -> None:
    """q_group [in, sum out] and scale_group [sum out] from the members' q
    [in, out_i] and scale [out_i] (projections that read one input)."""
    fn = "tern_group_gather"
    n = len(qs)
    if n != len(scales):
        raise ValueError(f"{fn}: {n} q matrices but {len(scales)} scales")
    n_in = qs[0].shape[0] if n else 0
    for i, (qi, si) in enumerate(zip(qs, scales)):
        if qi.dim() != 2:
            raise ValueError(f"{fn}: q[{i}] must be [in, out_i]")
        _need(fn, f"q[{i}]", qi, (n_in, qi.shape[1]), (torch.int8,))
        _need(fn, f"scale[{i}]", si, (qi.shape[1],), _F32)
    tot = sum(int(t.shape[1]) for t in qs)
    _need(fn, "q_group", q_group, (n_in, tot), (torch.int8,))
    _need(fn, "scale_group", scale_group, (tot,), _F32)
    _need_device(fn, *qs, *scales, q_group, scale_group)
    qa = (_vp * max(n, 1))(*[_ptr(t) for t in qs])
    sa = (_vp * max(n, 1))(*[_ptr(t) for t in scales])
    oa = (_i64 * max(n, 1))(*[int(t.shape[1]) for t in qs])
    rc = lib().tern_group_gather(qa, sa, oa, n, n_in, _ptr(q_group), _ptr(scale_group), _stream(stream))
    _check("tern_group_gather", rc)


def tern_scale_adamw(sgrad, scale, m, v, step: int, lr: float, scale_lr: float | None = None, b1: float = 0.9,
                     b2: float = 0.999, eps: float = 1e-8, wd: float = 0.0, stream=None) -> None:
    """AdamW step of the per-column scale from its gradient (in place on
    scale, m, v; scale_lr defaults to lr)."""
    fn = "tern_scale_adamw"
    if scale.dim() != 1:
        raise ValueError(f"{fn}: scale must be [out]")
    for name, t in (("sgrad", sgrad), ("scale", scale), ("m", m), ("v", v)):
        _need(fn, name, t, scale.shape, _F32)
    _need_device(fn, sgrad, scale, m, v)
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


def _need_panel(fn, panel):
    _need(fn, "panel", panel, (len(PANEL_COUNTS) + len(PANEL_STATS),), (torch.float64,))


def tern_panel_reset(panel: torch.Tensor, stream=None) -> None:
    _need_panel("tern_panel_reset", panel)
    _need_device("tern_panel_reset", panel)
    _check("tern_panel_reset", lib().tern_panel_reset(_ptr(panel), _stream(stream)))


def tern_panel_add(q: torch.Tensor, theta: int, scale: torch.Tensor, panel: torch.Tensor, prev_packed=None,
                   q_clamp: int = 7, stream=None) -> None:
    """Add one ternary matrix (q int8 [in, out], scale [out]) to the panel;
    prev_packed: the previous step's handle for churn, or None."""
    fn = "tern_panel_add"
    if q.dim() != 2:
        raise ValueError(f"{fn}: q must be [in, out]")
    n_in, n_out = q.shape
    _need(fn, "q", q, (n_in, n_out), (torch.int8,))
    _need(fn, "scale", scale, (n_out,), _F32)
    _need_panel(fn, panel)
    if prev_packed is not None:
        _need_packed(fn, prev_packed, n_in, n_out)
    _need_device(fn, q, scale, panel, prev_packed)
    rc = lib().tern_panel_add(_ptr(q), n_in, n_out, int(theta), int(q_clamp), _ptr(prev_packed), _ptr(scale),
                              _ptr(panel), _stream(stream))
    _check("tern_panel_add", rc)


PANEL_FRACTIONS = ("pct_neg", "pct_zero", "pct_pos", "rail_pct", "dead_pct", "churn_frac", "scale_mean")


def tern_panel_fractions(panel_host: torch.Tensor) -> dict:
    """The page's fractions of an accumulator (host copy), computed by the
    library's tern_panel_fractions."""
    h = panel_host.contiguous()
    if h.device.type != "cpu" or h.numel() != len(PANEL_COUNTS) + len(PANEL_STATS) or h.dtype != torch.float64:
        raise ValueError("tern_panel_fractions needs a host copy of one panel (12 x 8 bytes)")
    out = (ctypes.c_double * len(PANEL_FRACTIONS))()
    _check("tern_panel_fractions", lib().tern_panel_fractions(ctypes.c_void_p(h.data_ptr()), out))
    return dict(zip(PANEL_FRACTIONS, list(out)))


def panel_values(panel: torch.Tensor) -> dict:
    """The accumulator's fields (copied to the host) and the page's fractions
    of them from tern_panel_fractions."""
    h = panel.cpu()
    n = len(PANEL_COUNTS)
    r = dict(zip(PANEL_COUNTS, h[:n].view(torch.int64).tolist()))
    r.update(zip(PANEL_STATS, h[n:].tolist()))
    r.update(tern_panel_fractions(h))
    return r


class TernProj(ctypes.Structure):
    """tern_proj_t: one projection of a layer call."""
    _fields_ = [("in_", _i64), ("out", _i64), ("q", _vp), ("tern_packed", _vp), ("scale", _vp), ("X", _vp),
                ("dY", _vp), ("Y", _vp), ("dX", _vp), ("gq", _vp), ("sgrad", _vp)]


LAYER_MEMBERS = ("q", "packed", "scale", "X", "dY", "Y", "dX", "gq", "sgrad")


def _layer(fn: str, projs, T: int | None, need, act=None):
    """Marshal a list of projections (dicts with n_in, n_out and the device
    tensors the call uses: q, packed, scale, X, dY, Y, dX, gq, sgrad) into a
    tern_proj_t array, checking every tensor the call uses."""
    n = len(projs)
    if not 1 <= n <= 8:
        raise ValueError(f"{fn}: 1 to 8 projections, got {n}")
    arr = (TernProj * n)()
    used = []
    for i, d in enumerate(projs):
        ni, no = int(d["n_in"]), int(d["n_out"])
        shapes = {"q": ((ni, no), (torch.int8,)), "scale": ((no,), _F32), "X": ((T, ni), act),
                  "dY": ((T, no), act), "Y": ((T, no), (torch.float32, act[0] if act else None)),
                  "dX": ((T, ni), _F32), "gq": ((ni, no), _F32), "sgrad": ((no,), _F32)}
        for k in need:
            if k == "packed":
                _need_packed(fn, d.get("packed"), ni, no)
            else:
                shape, dts = shapes[k]
                _need(fn, f"{k}[{i}]", d.get(k), shape, dts)
            used.append(d.get(k))
        arr[i].in_, arr[i].out = ni, no
        for k, field in (("q", "q"), ("packed", "tern_packed"), ("scale", "scale"), ("X", "X"), ("dY", "dY"),
                         ("Y", "Y"), ("dX", "dX"), ("gq", "gq"), ("sgrad", "sgrad")):
            if k in need:
                p = _ptr(d[k])
                setattr(arr[i], field, p.value if p is not None else None)
    _need_device(fn, *used)
    return arr


def tern_layer_materialize(projs, theta: int, stream=None) -> None:
    """tern_materialize of every projection (q -> packed), one launch."""
    arr = _layer("tern_layer_materialize", projs, None, ("q", "packed"))
    _check("tern_layer_materialize", lib().tern_layer_materialize(arr, len(projs), int(theta), _stream(stream)))


def tern_layer_fwd(projs, stream=None) -> None:
    """tern_linear_fwd of every projection (they share T and X's dtype)."""
    X0 = projs[0]["X"]
    act = (X0.dtype,)
    arr = _layer("tern_layer_fwd", projs, X0.shape[0], ("packed", "scale", "X", "Y"), act)
    ydt = _act_code(projs[0]["Y"])
    if any(_act_code(d["Y"]) != ydt for d in projs):
        raise TypeError("tern_layer_fwd: every Y must have the same dtype")
    _check("tern_layer_fwd", lib().tern_layer_fwd(arr, len(projs), X0.shape[0], _act_code(X0), ydt, _stream(stream)))


def tern_layer_bwd_dx(projs, stream=None) -> None:
    """tern_linear_bwd_dx of every projection."""
    dY0 = projs[0]["dY"]
    arr = _layer("tern_layer_bwd_dx", projs, dY0.shape[0], ("packed", "scale", "dY", "dX"), (dY0.dtype,))
    _check("tern_layer_bwd_dx", lib().tern_layer_bwd_dx(arr, len(projs), dY0.shape[0], _act_code(dY0),
                                                       _stream(stream)))


def tern_layer_bwd_dw_workspace_bytes(shapes, T: int) -> int:
    """Workspace of tern_layer_bwd_dw for projections of these (n_in, n_out)."""
    n = len(shapes)
    arr = (TernProj * max(n, 1))()
    for i, (ni, no) in enumerate(shapes):
        arr[i].in_, arr[i].out = int(ni), int(no)
    return int(lib().tern_layer_bwd_dw_workspace_bytes(arr, n, int(T)))


def empty_layer_workspace(shapes, T: int, device="cuda") -> torch.Tensor:
    nbytes = tern_layer_bwd_dw_workspace_bytes(shapes, T)
    return torch.empty((max(nbytes, 16) // 16, 16), dtype=torch.uint8, device=device)


def tern_layer_bwd_dw(projs, workspace, stream=None) -> None:
    """tern_linear_bwd_dw of every projection (gq, sgrad)."""
    X0 = projs[0]["X"]
    arr = _layer("tern_layer_bwd_dw", projs, X0.shape[0], ("packed", "scale", "X", "dY", "gq", "sgrad"),
                 (X0.dtype,))
    _need_device("tern_layer_bwd_dw", workspace)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("tern_layer_bwd_dw", lib().tern_layer_bwd_dw(arr, len(projs), X0.shape[0], _act_code(X0),
                                                       _ptr(workspace), ws_bytes, _stream(stream)))


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


def empty_workspace(T: int, n_in: int, n_out: int, device="cuda", acc: bool = False) -> torch.Tensor:
    """Workspace of tern_linear_bwd / tern_linear_bwd_dw (acc: of
    tern_linear_bwd_dw_acc), for either activation type."""
    q = tern_linear_bwd_acc_workspace_bytes if acc else tern_linear_bwd_workspace_bytes
    nbytes = q(T, n_in, n_out)
    return torch.empty((max(nbytes, 16) // 16, 16), dtype=torch.uint8, device=device)
