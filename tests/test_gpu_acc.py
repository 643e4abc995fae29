"""Accumulating backward variants on the GPU, through the C ABI.

tern_linear_bwd_dx_acc adds dY . W_eff^T to dX; tern_linear_bwd_dw_acc adds
alpha * G * scale to gq and alpha * sum_r G * tern to sgrad.  They are held to
the oracle (the old value plus the oracle's result, and the increment alone),
and, bit for bit, to the plain entry points wherever fp32 arithmetic makes the
two equal: adding to zero, adding twice, and adding with a power-of-two alpha.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import ternary_weight_linear_tern_amd as tl
from gpu_util import DeviceProjection, check_elements, log, rel_l2, tol_for

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


def _like(ref: np.ndarray, seed: int) -> torch.Tensor:
    """A seeded fp32 tensor of ref's shape and RMS (the old value to add to)."""
    g = torch.Generator().manual_seed(seed)
    rms = float(np.sqrt(np.mean(np.square(ref)))) if ref.size else 1.0
    return (torch.randn(ref.shape, generator=g, dtype=torch.float64) * rms).float().cuda()


def _acc_dw(d, gq, sg, alpha):
    ws = tl.empty_workspace(d.T, d.n_in, d.n_out, acc=True)
    tl.tern_linear_bwd_dw_acc(d.X, d.dY, d.packed, d.scale, gq, sg, ws, alpha)


@pytest.mark.parametrize("T,n_in,n_out,act", [(64, 64, 64, "f32"), (129, 72, 136, "bf16"),
                                              (300, 200, 520, "bf16"), (1000, 256, 264, "f32"),
                                              (777, 136, 1032, "bf16")])
@pytest.mark.parametrize("alpha", [1.0, 1.0 / 3.0])
def test_acc_matches_oracle(o, T, n_in, n_out, act, alpha):
    log(f"accumulate vs oracle T={T} in={n_in} out={n_out} {act} alpha={alpha:.4f}")
    p = synth.make_inputs(T, n_in, n_out, act=act, config_id=800)
    d = DeviceProjection(p)
    d.materialize()
    dXo = o.linear_dx(p.dY, p.q, p.theta, p.scale)
    _, gqo, sgo = o.linear_wgrad(p.X, p.dY, p.q, p.theta, p.scale)
    dX0, gq0, sg0 = _like(dXo, 1), _like(gqo, 2), _like(sgo, 3)
    dX, gq, sg = dX0.clone(), gq0.clone(), sg0.clone()
    tl.tern_linear_bwd_dx_acc(d.dY, d.packed, d.scale, dX)
    _acc_dw(d, gq, sg, alpha)
    torch.cuda.synchronize()
    f64 = lambda t: t.cpu().numpy().astype(np.float64)
    tol = tol_for(act)
    errs = dict(
        dX=rel_l2(f64(dX), f64(dX0) + dXo), gq=rel_l2(f64(gq), f64(gq0) + alpha * gqo),
        sgrad=rel_l2(f64(sg), f64(sg0) + alpha * sgo),
        # the increments alone (the old values have the increments' size, so
        # the final fp32 add costs at most a few 2^-24)
        d_dX=rel_l2(f64(dX) - f64(dX0), dXo), d_gq=rel_l2(f64(gq) - f64(gq0), alpha * gqo),
        d_sgrad=rel_l2(f64(sg) - f64(sg0), alpha * sgo))
    log(f"  relL2 {errs}")
    for k, e in errs.items():
        assert e <= tol, f"{k} relL2 {e:.3e} > {tol:.1e}"
    # each increment element within its own rounding bound, plus the final fp32
    # add's rounding (at most 2^-24 of the stored value, counted twice for slack)
    olds = dict(dX=f64(dX0), gq=f64(gq0), sgrad=f64(sg0))
    news = dict(dX=f64(dX), gq=f64(gq), sgrad=f64(sg))
    scale = dict(dX=1.0, gq=alpha, sgrad=alpha)
    inc = {k: (news[k] - olds[k]) / scale[k] for k in olds}
    slack = {k: 2.0 ** -23 * (np.abs(olds[k]) + np.abs(news[k])) / scale[k] for k in olds}
    check_elements(o, p, inc, dict(dX=dXo, gq=gqo, sgrad=sgo), tag=f"accumulate T={T} in={n_in} out={n_out}",
                   slack=slack)


@pytest.mark.parametrize("T,n_in,n_out", [(4000, 1032, 4104), (4000, 4104, 1032), (2048, 512, 2048)])
def test_acc_bitwise_against_plain(o, T, n_in, n_out):
    """256-tile (persistent) kernels, ragged edges: the accumulating calls give
    exactly old + plain in fp32, and their increments meet the oracle on
    sampled rows and columns."""
    log(f"accumulate bitwise T={T} in={n_in} out={n_out}")
    p = synth.make_inputs(T, n_in, n_out, act="bf16", config_id=810, proj_id=n_in)
    d = DeviceProjection(p)
    d.step()
    torch.cuda.synchronize()
    dX_plain, gq_plain, sg_plain = d.dX.clone(), d.gq.clone(), d.sgrad.clone()

    # dX: onto zero, then once more (v + v = 2v exactly), then onto old values
    dX = torch.zeros_like(dX_plain)
    tl.tern_linear_bwd_dx_acc(d.dY, d.packed, d.scale, dX)
    torch.cuda.synchronize()
    assert torch.equal(dX, dX_plain), "dX accumulated onto zero differs from the plain dX"
    tl.tern_linear_bwd_dx_acc(d.dY, d.packed, d.scale, dX)
    torch.cuda.synchronize()
    assert torch.equal(dX, 2 * dX_plain), "second accumulation differs from 2 dX"
    dX0 = _like(dX_plain.cpu().numpy(), 11)
    dX = dX0.clone()
    tl.tern_linear_bwd_dx_acc(d.dY, d.packed, d.scale, dX)
    torch.cuda.synchronize()
    assert torch.equal(dX, dX0 + dX_plain), "dX += differs from old + plain in fp32"

    # gq, sgrad with alpha = 1/4 (alpha * t is exact, so fused or not the add rounds once)
    gq0 = _like(gq_plain.cpu().numpy(), 12)
    sg0 = _like(sg_plain.cpu().numpy(), 13)
    gq, sg = gq0.clone(), sg0.clone()
    _acc_dw(d, gq, sg, 0.25)
    torch.cuda.synchronize()
    assert torch.equal(gq, gq0 + 0.25 * gq_plain), "gq += differs from old + alpha plain in fp32"
    e_sg = rel_l2(sg.cpu().numpy(), sg0.cpu().numpy().astype(np.float64) + 0.25 * sg_plain.cpu().numpy())
    assert e_sg <= 1e-6, f"sgrad += against old + alpha plain: relL2 {e_sg:.3e}"

    # the increments against the oracle on sampled token rows / output columns
    rows = np.union1d(synth.sample_indices(synth.stream_seed(79, T, n_in, 0), 32, T), [0, T - 1])
    cols = np.union1d(synth.sample_indices(synth.stream_seed(79, T, n_out, 1), 12, n_out), [0, n_out - 1])
    rt, ct = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    f64 = lambda t: t.cpu().numpy().astype(np.float64)
    _, gqo, sgo = o.linear_wgrad(p.X, p.dY, p.q, p.theta, p.scale, cols=cols)
    errs = dict(dX=rel_l2(f64(dX[rt]) - f64(dX0[rt]), o.linear_dx(p.dY, p.q, p.theta, p.scale, rows=rows)),
                gq=rel_l2((f64(gq[:, ct]) - f64(gq0[:, ct])) * 4.0, gqo),
                sgrad=rel_l2((f64(sg[ct]) - f64(sg0[ct])) * 4.0, sgo))
    log(f"  increments relL2 {errs}")
    for k, e in errs.items():
        assert e <= tol_for("bf16"), f"{k} increment relL2 {e:.3e}"


def test_acc_empty_sums_leave_outputs():
    """Nothing to add: dX with out = 0, gq / sgrad with T = 0 stay as they were
    (the plain calls would write zeros)."""
    dev = "cuda"
    dY = torch.empty((16, 0), dtype=torch.bfloat16, device=dev)
    sc0 = torch.empty((0,), device=dev)
    pk = tl.empty_packed(64, 8)
    dX = torch.full((16, 64), 3.0, device=dev)
    tl.tern_linear_bwd_dx_acc(dY, pk, sc0, dX, n_in=64)
    X = torch.empty((0, 64), dtype=torch.bfloat16, device=dev)
    dY2 = torch.empty((0, 32), dtype=torch.bfloat16, device=dev)
    q = torch.full((64, 32), 3, dtype=torch.int8, device=dev)
    sc = torch.ones(32, device=dev)
    pk2 = tl.empty_packed(64, 32)
    tl.tern_materialize(q, 2, pk2)
    gq = torch.full((64, 32), 5.0, device=dev)
    sg = torch.full((32,), 7.0, device=dev)
    ws = tl.empty_workspace(0, 64, 32, acc=True)
    tl.tern_linear_bwd_dw_acc(X, dY2, pk2, sc, gq, sg, ws, 0.5)
    torch.cuda.synchronize()
    assert bool((dX == 3.0).all()) and bool((gq == 5.0).all()) and bool((sg == 7.0).all())
