"""Projections that read one input, run as one projection over their
concatenated columns (tern_group_gather + the single-projection entry points),
on the GPU through the C ABI.

The group's q and scale are the members' side by side; its packing is the
oracle's packing of that concatenation; each member's column slice of the
group's Y equals that member's own forward bit for bit; the group's dX meets
the gate against the sum of the members' oracle input gradients, and the
gq / sgrad slices against each member's oracle weight-side gradients.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
import ternary_weight_linear_tern_amd as tl
from gpu_util import check_elements, log, rel_l2, to_dev, tol_for

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


def _members(T, n_in, outs, act, cid):
    ps = [synth.make_inputs(T, n_in, w, act=act, config_id=cid, proj_id=k) for k, w in enumerate(outs)]
    X = ps[0].X   # one input shared by every member
    return X, ps


def _run_group(X, ps, theta):
    T, n_in = X.shape
    tot = sum(p.q.shape[1] for p in ps)
    qs = [to_dev(p.q) for p in ps]
    ss = [to_dev(p.scale) for p in ps]
    qg = torch.empty((n_in, tot), dtype=torch.int8, device="cuda")
    sg = torch.empty((tot,), dtype=torch.float32, device="cuda")
    tl.tern_group_gather(qs, ss, qg, sg)
    Xd = to_dev(X)
    dYg = to_dev(np.concatenate([p.dY for p in ps], axis=1))
    pk = tl.empty_packed(n_in, tot)
    tl.tern_materialize(qg, theta, pk)
    Y = torch.empty((T, tot), device="cuda")
    dX = torch.empty((T, n_in), device="cuda")
    gq = torch.empty((n_in, tot), device="cuda")
    sgr = torch.empty((tot,), device="cuda")
    ws = tl.empty_workspace(T, n_in, tot)
    tl.tern_linear_fwd(Xd, pk, sg, Y)
    tl.tern_linear_bwd(Xd, dYg, pk, sg, dX, gq, sgr, ws)
    torch.cuda.synchronize()
    return dict(q=qg, scale=sg, packed=pk, Y=Y, dX=dX, gq=gq, sgrad=sgr, Xd=Xd)


def _member_fwd(Xd, p, theta):
    n_in, w = p.q.shape
    pk = tl.empty_packed(n_in, w)
    tl.tern_materialize(to_dev(p.q), theta, pk)
    Y = torch.empty((Xd.shape[0], w), device="cuda")
    tl.tern_linear_fwd(Xd, pk, to_dev(p.scale), Y)
    torch.cuda.synchronize()
    return Y


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_group_matches_members(o, act):
    T, n_in, outs = 1000, 264, [136, 264, 520]
    log(f"group of {outs} sharing X [{T}, {n_in}] ({act})")
    X, ps = _members(T, n_in, outs, act, 850)
    theta = ps[0].theta
    g = _run_group(X, ps, theta)
    q_cat = np.concatenate([p.q for p in ps], axis=1)
    assert np.array_equal(g["q"].cpu().numpy(), q_cat), "gathered q differs from the concatenation"
    assert np.array_equal(g["scale"].cpu().numpy(), np.concatenate([p.scale for p in ps])), "gathered scale"
    pk = tl.packed_canonical(g["packed"], n_in, sum(outs)).cpu().numpy().view(np.uint32)
    assert np.array_equal(pk, o.pack(o.tern(q_cat, theta))), "group packing differs from the oracle"
    tol = tol_for(act)
    dX_want = sum(o.linear_dx(p.dY, p.q, theta, p.scale) for p in ps)
    e = rel_l2(g["dX"].cpu().numpy(), dX_want)
    log(f"  dX (sum over members) relL2 {e:.3e}")
    assert e <= tol
    off = 0
    for k, p in enumerate(ps):
        w = p.q.shape[1]
        Yk = _member_fwd(g["Xd"], p, theta)
        assert torch.equal(g["Y"][:, off:off + w], Yk), f"member {k}: Y slice differs from its own forward"
        assert rel_l2(Yk.cpu().numpy(), o.linear_fwd(X, p.q, theta, p.scale)) <= tol
        _, gqo, sgo = o.linear_wgrad(X, p.dY, p.q, theta, p.scale)
        eg = rel_l2(g["gq"][:, off:off + w].cpu().numpy(), gqo)
        es = rel_l2(g["sgrad"][off:off + w].cpu().numpy(), sgo)
        log(f"  member {k}: gq relL2 {eg:.3e} sgrad relL2 {es:.3e}")
        assert eg <= tol and es <= tol
        # the member's slices element by element within their rounding bounds
        check_elements(o, dataclasses.replace(p, X=X), dict(Y=g["Y"][:, off:off + w].cpu().numpy(), gq=g["gq"][:, off:off + w].cpu().numpy(),
                                  sgrad=g["sgrad"][off:off + w].cpu().numpy()),
                       dict(Y=o.linear_fwd(X, p.q, theta, p.scale), gq=gqo, sgrad=sgo), tag=f"group member {k}")
        off += w


def test_group_qkv_large_sampled(o):
    """A fused q/k/v at d = 2048 (three 2048 -> 2048 members, T = 4096): the
    256-tile kernels; Y slices bitwise equal to each member's forward, dX and
    gq / sgrad against the oracle on sampled rows and columns."""
    T, n_in, outs = 4096, 2048, [2048, 2048, 2048]
    log("group q/k/v d=2048")
    X, ps = _members(T, n_in, outs, "bf16", 860)
    theta = ps[0].theta
    g = _run_group(X, ps, theta)
    rows = np.union1d(synth.sample_indices(synth.stream_seed(81, T, n_in, 0), 24, T), [0, T - 1])
    rt = torch.from_numpy(rows).cuda()
    dX_want = sum(o.linear_dx(p.dY, p.q, theta, p.scale, rows=rows) for p in ps)
    e = rel_l2(g["dX"][rt].cpu().numpy(), dX_want)
    log(f"  dX relL2 {e:.3e}")
    assert e <= tol_for("bf16")
    off = 0
    for k, p in enumerate(ps):
        w = p.q.shape[1]
        assert torch.equal(g["Y"][:, off:off + w], _member_fwd(g["Xd"], p, theta)), f"member {k} Y slice"
        cols = np.union1d(synth.sample_indices(synth.stream_seed(81, T, w, k + 1), 6, w), [0, w - 1])
        ct = torch.from_numpy(cols + off).cuda()
        _, gqo, sgo = o.linear_wgrad(X, p.dY, p.q, theta, p.scale, cols=cols)
        eg = rel_l2(g["gq"][:, ct].cpu().numpy(), gqo)
        es = rel_l2(g["sgrad"][ct].cpu().numpy(), sgo)
        log(f"  member {k}: gq {eg:.3e} sgrad {es:.3e}")
        assert eg <= tol_for("bf16") and es <= tol_for("bf16")
        off += w
