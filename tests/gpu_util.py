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
        self.ws = tl.empty_workspace(T, n_in, n_out, self.X.dtype)

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
