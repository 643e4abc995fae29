"""Scales of either sign and exact zeros, through the C ABI on the GPU.

The trainer updates scale with AdamW and weight decay (page "train_gpu.cu",
the optimizer-split header comment), so nothing keeps a scale positive: it
can reach zero or cross it.  W_eff = scale[c] * tern[r, c] holds for any
sign, so every output must still meet the oracle:
* the forward multiplies its column sums by the signed scale in the epilogue;
* dX carries +-bf16(scale[c]) in its operand (or the two-term split where the
  fold is not exact enough), built by flipping the sign bit of the scale's
  bf16 pattern for tern = -1, which must not assume a positive scale;
* gq = G * scale[c] and sgrad, which does not depend on scale at all.

Shapes cover the persistent kernels (ragged, dW split over tokens),
the two-term dX scale (few columns), the fp32 path and the layer calls.
Columns with scale 0 give exactly zero Y and gq columns and no dX
contribution.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import ternary_weight_linear_tern_amd as tl
from gpu_util import DeviceProjection, check_elements, log, rel_l2, to_dev, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    tl.lib()
    yield
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def o():
    return oracle.get()


def _signed(p, seed):
    """The inputs' scale with random signs and about one column in eight set to 0."""
    rng = np.random.default_rng(seed)
    n = p.scale.shape[0]
    sign = np.where(rng.random(n) < 0.5, -1.0, 1.0).astype(np.float32)
    zero = rng.random(n) < 0.125
    zero[0] = True   # at least one zero column
    p.scale = np.where(zero, np.float32(0.0), sign * p.scale).astype(np.float32)
    return zero


@pytest.mark.parametrize("T,n_in,n_out,act", [(4000, 1032, 1032, "bf16"), (2056, 2056, 2056, "bf16"),
                                              (520, 264, 40, "bf16"), (1000, 264, 136, "f32")])
def test_signed_scale(o, T, n_in, n_out, act):
    log(f"signed scale {T}x{n_in}x{n_out} {act}")
    p = synth.make_inputs(T, n_in, n_out, act=act, config_id=1901)
    zero = _signed(p, 1901)
    d = DeviceProjection(p)
    d.step()
    r = d.results()
    Y = o.linear_fwd(p.X, p.q, p.theta, p.scale)
    dX = o.linear_dx(p.dY, p.q, p.theta, p.scale)
    _, gq, sg = o.linear_wgrad(p.X, p.dY, p.q, p.theta, p.scale)
    tol = tol_for(act)
    errs = {k: rel_l2(r[k], w) for k, w in (("Y", Y), ("dX", dX), ("gq", gq), ("sgrad", sg))}
    log("  relL2 " + ", ".join(f"{k} {v:.3e}" for k, v in errs.items()))
    for k, e in errs.items():
        assert e <= tol, f"{k} relL2 {e:.3e} above {tol:.0e} with signed scales"
    check_elements(o, p, {k: r[k] for k in ("Y", "dX", "gq", "sgrad")},
                   {"Y": Y, "dX": dX, "gq": gq, "sgrad": sg}, tag=f"signed scale {T}x{n_in}x{n_out}")
    # a zero scale zeroes its whole column of W_eff
    assert np.all(r["Y"][:, zero] == 0.0), "Y column of a zero scale is not exactly zero"
    assert np.all(r["gq"][:, zero] == 0.0), "gq column of a zero scale is not exactly zero"


def test_signed_scale_layer(o):
    """The layer calls with signed and zero scales, against the oracle on sampled rows and columns."""
    T = 2048
    shapes = [(1024, 1024), (1024, 4096), (4096, 1024)]
    log("signed scale, layer calls")
    projs, host = [], []
    for i, (ni, no) in enumerate(shapes):
        p = synth.make_inputs(T, ni, no, act="bf16", config_id=1902, proj_id=i)
        _signed(p, 1902 + i)
        projs.append(dict(n_in=ni, n_out=no, q=to_dev(p.q), scale=to_dev(p.scale), X=to_dev(p.X),
                          dY=to_dev(p.dY), packed=tl.empty_packed(ni, no), Y=torch.empty((T, no), device="cuda"),
                          dX=torch.empty((T, ni), device="cuda"), gq=torch.empty((ni, no), device="cuda"),
                          sgrad=torch.empty((no,), device="cuda")))
        host.append(p)
    ws = tl.empty_layer_workspace(shapes, T)
    tl.tern_layer_materialize(projs, 2)
    tl.tern_layer_fwd(projs)
    tl.tern_layer_bwd_dx(projs)
    tl.tern_layer_bwd_dw(projs, ws)
    torch.cuda.synchronize()
    for i, (d, p) in enumerate(zip(projs, host)):
        r = synth.sample_indices(700 + i, 32, T)
        c = synth.sample_indices(800 + i, 16, d["n_out"])
        got = {"Y": d["Y"].cpu().numpy()[r], "dX": d["dX"].cpu().numpy()[r]}
        want = {"Y": o.linear_fwd(p.X, p.q, p.theta, p.scale, rows=r),
                "dX": o.linear_dx(p.dY, p.q, p.theta, p.scale, rows=r)}
        _, gq, sg = o.linear_wgrad(p.X, p.dY, p.q, p.theta, p.scale, cols=c)
        got["gq"], got["sgrad"] = d["gq"].cpu().numpy()[:, c], d["sgrad"].cpu().numpy()[c]
        want["gq"], want["sgrad"] = gq, sg
        for k in got:
            e = rel_l2(got[k], want[k])
            assert e <= 2e-3, f"layer projection {i}: {k} relL2 {e:.3e} with signed scales"
        check_elements(o, p, {"Y": got["Y"], "dX": got["dX"]}, {"Y": want["Y"], "dX": want["dX"]}, rows=r,
                       tag=f"signed scale layer {i}")
        check_elements(o, p, {"gq": got["gq"], "sgrad": got["sgrad"]}, {"gq": gq, "sgrad": sg}, cols=c,
                       tag=f"signed scale layer {i} dW")
