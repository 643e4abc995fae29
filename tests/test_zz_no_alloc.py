"""tern_linear_bwd_noalloc against tern_linear_bwd, through the C ABI.

Two calls in a row on one GPU share the library's static scratch; the second
has a smaller input.  Where both entry points plan the same split of the
weight-gradient product the outputs are bitwise equal; where the static
scratch forces fewer splits (the d = 2048 shapes at 16384 tokens) they agree
to the bf16 gate and meet the oracle on sampled columns and rows.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import ternary_weight_linear_tern_amd as tl
from gpu_util import DeviceProjection, log, rel_l2, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    tl.lib()
    yield
    torch.cuda.synchronize()


def _run_both(p):
    d = DeviceProjection(p)
    d.materialize()
    d.bwd()
    ref = dict(dX=d.dX.clone(), gq=d.gq.clone(), sgrad=d.sgrad.clone())
    d.dX.fill_(float("nan"))
    d.gq.fill_(float("nan"))
    d.sgrad.fill_(float("nan"))
    tl.tern_linear_bwd_noalloc(d.X, d.dY, d.packed, d.scale, d.dX, d.gq, d.sgrad)
    torch.cuda.synchronize()
    got = dict(dX=d.dX.clone(), gq=d.gq.clone(), sgrad=d.sgrad.clone())
    return d, ref, got


def _bitwise(ref, got, tag):
    for k in ref:
        assert torch.equal(ref[k], got[k]), f"{tag}: {k} differs from tern_linear_bwd"


def test_noalloc_two_calls_smaller_second():
    o = oracle.get()
    # first call: the static scratch holds fewer splits than the usual plan
    p1 = synth.make_inputs(16384, 2048, 2048, act="bf16", config_id=1501)
    log("noalloc call 1: 16384 x 2048 x 2048 (fewer splits than tern_linear_bwd)")
    d1, ref1, got1 = _run_both(p1)
    _bitwise({"dX": ref1["dX"]}, {"dX": got1["dX"]}, "call 1")   # dX takes no scratch
    for k in ("gq", "sgrad"):
        e = rel_l2(got1[k].cpu().numpy(), ref1[k].cpu().numpy())
        log(f"  {k} relL2 against tern_linear_bwd {e:.3e}")
        assert e <= 1e-5, f"{k}: {e:.3e}"
    cols = synth.sample_indices(77, 12, 2048)
    _, gqo, sgo = o.linear_wgrad(p1.X, p1.dY, p1.q, p1.theta, p1.scale, cols=cols)
    assert rel_l2(got1["gq"].cpu().numpy()[:, cols], gqo) <= 2e-3
    assert rel_l2(got1["sgrad"].cpu().numpy()[cols], sgo) <= 2e-3
    del d1
    # second call, smaller: the same plan as tern_linear_bwd, bitwise equal
    for shape, act in (((4000, 1032, 1032), "bf16"), ((300, 136, 264), "bf16"), ((200, 64, 96), "f32")):
        log(f"noalloc call: {shape} {act}")
        p = synth.make_inputs(*shape, act=act, config_id=1502)
        _, ref, got = _run_both(p)
        _bitwise(ref, got, f"{shape} {act}")
        want = o.linear_dx(p.dY, p.q, p.theta, p.scale)
        assert rel_l2(got["dX"].cpu().numpy(), want) <= (2e-3 if act == "bf16" else 1e-5)


def test_noalloc_zero_sizes():
    dev = "cuda"
    X = torch.empty((0, 64), dtype=torch.bfloat16, device=dev)
    dY = torch.empty((0, 32), dtype=torch.bfloat16, device=dev)
    q = torch.full((64, 32), 3, dtype=torch.int8, device=dev)
    sc = torch.ones(32, device=dev)
    pk = tl.empty_packed(64, 32)
    tl.tern_materialize(q, 2, pk)
    dX = torch.empty((0, 64), device=dev)
    gq = torch.full((64, 32), 7.0, device=dev)
    sg = torch.full((32,), 7.0, device=dev)
    tl.tern_linear_bwd_noalloc(X, dY, pk, sc, dX, gq, sg)
    torch.cuda.synchronize()
    assert bool((gq == 0).all()) and bool((sg == 0).all())
