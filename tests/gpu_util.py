"""Helpers of the GPU parity tests: move seeded inputs to the device, run the
HIP path through the C ABI, compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import ternary_weight_linear_tern_amd as tl

TOL_BF16 = 2e-3   # rel-L2 gate for bf16 activations
TOL_F32 = 1e-5    # rel-L2 gate for fp32 activations


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    """numpy input -> device tensor; uint16 arrays carry bf16 bits."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def rel_l2(a, ref) -> float:
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert a.shape == ref.shape, (a.shape, ref.shape)
    nr = float(np.linalg.norm(ref))
    if nr == 0.0:
        return 0.0 if not np.any(a) else float("inf")
    return float(np.linalg.norm(a - ref) / nr)


def tol_for(act: str) -> float:
    return TOL_BF16 if act == "bf16" else TOL_F32


class DeviceProjection:
    """Device copies of one projection's inputs and its outputs."""

    def __init__(self, p, y_bf16: bool = False):
        self.p = p
        T, n_in = p.X.shape
        n_out = p.q.shape[1]
        self.T, self.n_in, self.n_out = T, n_in, n_out
        self.X = to_dev(p.X)
        self.dY = to_dev(p.dY)
        self.q = to_dev(p.q)
        self.scale = to_dev(p.scale)
        self.packed = tl.empty_packed(n_in, n_out)
        ydt = torch.bfloat16 if y_bf16 else torch.float32
        self.Y = torch.empty((T, n_out), dtype=ydt, device="cuda")
        self.dX = torch.empty((T, n_in), dtype=torch.float32, device="cuda")
        self.gq = torch.empty((n_in, n_out), dtype=torch.float32, device="cuda")
        self.sgrad = torch.empty((n_out,), dtype=torch.float32, device="cuda")
        self.ws = tl.empty_workspace(T, n_in, n_out)

    def materialize(self, theta=None):
        tl.tern_materialize(self.q, self.p.theta if theta is None else theta, self.packed)

    def fwd(self):
        tl.tern_linear_fwd(self.X, self.packed, self.scale, self.Y)

    def bwd(self):
        tl.tern_linear_bwd(self.X, self.dY, self.packed, self.scale, self.dX, self.gq, self.sgrad, self.ws)

    def step(self):
        self.materialize()
        self.fwd()
        self.bwd()

    def results(self) -> dict:
        torch.cuda.synchronize()
        Y = self.Y.float() if self.Y.dtype == torch.bfloat16 else self.Y
        pk = tl.packed_canonical(self.packed, self.n_in, self.n_out)
        return dict(packed=pk.cpu().numpy().view(np.uint32), Y=Y.cpu().numpy(),
                    dX=self.dX.cpu().numpy(), gq=self.gq.cpu().numpy(), sgrad=self.sgrad.cpu().numpy())


def _abs_act(a: np.ndarray) -> np.ndarray:
    """|a| for an activation array (bf16 bit patterns: clear the sign bit)."""
    return a & np.uint16(0x7FFF) if a.dtype == np.uint16 else np.abs(a)


def check_elements(o, p, got, want, rows=None, cols=None, tag="", slack=None):
    """Each element within its own rounding bound.

    With the inputs exact in both computations, the device result differs from
    the oracle's f64 value only by the roundings of its fp32 sums and of the
    operand it rounds:  |got - want| <= (u_op + 2 (K + 2) 2^-24) * S,  where
    S = sum |a| |b| over the element's products (the oracle's own product of
    the absolute values), K the length of that sum (in for Y, out for dX, T for
    gq and sgrad) plus the fp32 sums added on top of it: up to 32 split
    partials of G (gq), and for sgrad also the in-tile sum over a 256-row tile
    (64 sequential adds in a lane, then the lane pair and the two waves: 66,
    counted as 33 since the formula doubles K), so K = T + 32 for gq and
    T + 32 + 33 for sgrad; u_op = 2^-8 for dX with bf16 activations (its scale is
    rounded to bf16 inside the operand), else 0.  A misplaced or stale element
    is off by about sqrt(K) typical terms, far beyond this bound, even where
    one element barely moves the relative L2 norm.  slack: optional per-output
    arrays added to the bound (the rounding of a further fp32 operation).
    """
    T, n_in = p.X.shape
    n_out = p.q.shape[1]
    aX, adY = _abs_act(p.X), _abs_act(p.dY)
    aq = np.minimum(np.abs(p.q.astype(np.int16)), 127).astype(np.int8)
    asc = np.abs(p.scale)
    S = {}
    if "Y" in got:
        S["Y"] = o.linear_fwd(aX, aq, p.theta, asc, rows=rows)
    if "dX" in got:
        S["dX"] = o.linear_dx(adY, aq, p.theta, asc, rows=rows)
    if "gq" in got or "sgrad" in got:
        _, S["gq"], S["sgrad"] = o.linear_wgrad(aX, adY, aq, p.theta, asc, cols=cols)
    u_op = dict(Y=0.0, dX=2.0 ** -8 if p.act == "bf16" else 0.0, gq=0.0, sgrad=0.0)
    K = dict(Y=n_in, dX=n_out, gq=T + 32, sgrad=T + 32 + 33)
    for k in [k for k in ("Y", "dX", "gq", "sgrad") if k in got]:
        err = np.abs(np.asarray(got[k], dtype=np.float64) - want[k])
        bound = (u_op[k] + 2.0 * (K[k] + 2) * 2.0 ** -24) * S[k] + 1e-30
        if slack is not None and k in slack:
            bound = bound + slack[k]
        bad = np.argwhere(err > bound)
        if bad.size:
            i = tuple(bad[0])
            raise AssertionError(f"{tag}: {k}{list(i)} off by {err[i]:.3e} > bound {bound[i]:.3e} "
                                 f"({bad.shape[0]} elements out of bound)")
