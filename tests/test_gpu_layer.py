"""The layer calls (tern_layer_*, one launch per product for all projections)
against the single-projection calls and the oracle, through the C ABI.

* Packing, Y and dX equal the single-projection results bit for bit (the same
  tiles in the same order, only walked by one grid); gq and sgrad, whose split
  over tokens is planned for the layer, agree to fp32 rounding and meet the
  oracle's gate.
* Layers mixing projections the grouped kernels take with ones they do not
  (a dW side below 256, a dX with the exact two-term scale, fp32 activations,
  an empty projection) give the same results as the single calls.
* A shared input (one X for three projections) and repeated calls (bitwise
  equal).
* The d = 1024 block at 8192 tokens, whose forward and dX mix items of 128
  and 32 chunks: the planner walks them in two classes of workgroups (the
  planner check on the CPU pins that choice); the results equal the
  single-projection calls bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import ternary_weight_linear_tern_amd as tl
from gpu_util import log, rel_l2, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    tl.lib()
    yield
    torch.cuda.synchronize()


def _make(T, shapes, act="bf16", config_id=1600, shared_x=False):
    projs, host = [], []
    X_shared = None
    for i, (ni, no) in enumerate(shapes):
        p = synth.make_inputs(T, ni, no, act=act, config_id=config_id, proj_id=i)
        if shared_x:
            if X_shared is None:
                X_shared = p.X
            p.X = X_shared
        d = dict(n_in=ni, n_out=no, q=to_dev(p.q), scale=to_dev(p.scale), X=to_dev(p.X), dY=to_dev(p.dY),
                 packed=tl.empty_packed(ni, no), Y=torch.empty((T, no), device="cuda"),
                 dX=torch.empty((T, ni), device="cuda"), gq=torch.empty((ni, no), device="cuda"),
                 sgrad=torch.empty((no,), device="cuda"))
        if shared_x and i > 0:
            d["X"] = projs[0]["X"]
        projs.append(d)
        host.append(p)
    return projs, host


def _single(projs, theta=2):
    out = []
    for d in projs:
        pk = tl.empty_packed(d["n_in"], d["n_out"])
        tl.tern_materialize(d["q"], theta, pk)
        Y = torch.empty_like(d["Y"])
        dX = torch.empty_like(d["dX"])
        gq = torch.empty_like(d["gq"])
        sg = torch.empty_like(d["sgrad"])
        tl.tern_linear_fwd(d["X"], pk, d["scale"], Y)
        tl.tern_linear_bwd_dx(d["dY"], pk, d["scale"], dX)
        tl.tern_linear_bwd_dw(d["X"], d["dY"], pk, d["scale"], gq, sg, tl.empty_workspace(
            d["X"].shape[0], d["n_in"], d["n_out"]))
        out.append(dict(packed=pk, Y=Y, dX=dX, gq=gq, sgrad=sg))
    torch.cuda.synchronize()
    return out


def _layer(projs, theta=2):
    T = projs[0]["X"].shape[0]
    ws = tl.empty_layer_workspace([(d["n_in"], d["n_out"]) for d in projs], T)
    tl.tern_layer_materialize(projs, theta)
    tl.tern_layer_fwd(projs)
    tl.tern_layer_bwd_dx(projs)
    tl.tern_layer_bwd_dw(projs, ws)
    torch.cuda.synchronize()


def _compare(projs, ref, tag, dw_bitwise=False):
    for i, (d, r) in enumerate(zip(projs, ref)):
        words = tl.tern_packed_words(d["n_in"], d["n_out"])
        assert torch.equal(d["packed"][:words], r["packed"][:words]), f"{tag}[{i}]: handle differs"
        assert torch.equal(d["Y"], r["Y"]), f"{tag}[{i}]: Y differs from tern_linear_fwd"
        assert torch.equal(d["dX"], r["dX"]), f"{tag}[{i}]: dX differs from tern_linear_bwd_dx"
        for k in ("gq", "sgrad"):
            if dw_bitwise:
                assert torch.equal(d[k], r[k]), f"{tag}[{i}]: {k} differs"
            else:
                e = rel_l2(d[k].cpu().numpy(), r[k].cpu().numpy())
                assert e <= 1e-5, f"{tag}[{i}]: {k} relL2 {e:.3e} against tern_linear_bwd_dw"


def _oracle_check(projs, host, tag, rows=24, cols=12):
    o = oracle.get()
    for i, (d, p) in enumerate(zip(projs, host)):
        T = p.X.shape[0]
        r = synth.sample_indices(500 + i, rows, T)
        c = synth.sample_indices(600 + i, cols, d["n_out"])
        tol = 2e-3 if p.act == "bf16" else 1e-5
        assert rel_l2(d["Y"].cpu().numpy()[r], o.linear_fwd(p.X, p.q, p.theta, p.scale, rows=r)) <= tol
        assert rel_l2(d["dX"].cpu().numpy()[r], o.linear_dx(p.dY, p.q, p.theta, p.scale, rows=r)) <= tol
        _, gq, sg = o.linear_wgrad(p.X, p.dY, p.q, p.theta, p.scale, cols=c)
        assert rel_l2(d["gq"].cpu().numpy()[:, c], gq) <= tol, f"{tag}[{i}] gq"
        assert rel_l2(d["sgrad"].cpu().numpy()[c], sg) <= tol, f"{tag}[{i}] sgrad"


def test_layer_rwkv_small_block():
    """The RWKV small block: four 512 x 512, 512 -> 2048, 2048 -> 512 at 2048 tokens."""
    shapes = [(512, 512)] * 4 + [(512, 2048), (2048, 512)]
    projs, host = _make(2048, shapes, config_id=1601)
    ref = _single(projs)
    _layer(projs)
    _compare(projs, ref, "rwkv_small")
    _oracle_check(projs, host, "rwkv_small")
    log("  layer rwkv_small: equal to the single calls, oracle gate met")


def test_layer_repeatable_and_split_dw():
    """Larger dW products (split over tokens in the layer plan): two calls are
    bitwise identical."""
    shapes = [(1032, 1032), (1024, 2048), (2048, 1032)]
    projs, host = _make(4000, shapes, config_id=1602)
    ref = _single(projs)
    _layer(projs)
    first = [dict(gq=d["gq"].clone(), sgrad=d["sgrad"].clone()) for d in projs]
    _compare(projs, ref, "split")
    _layer(projs)
    for a, d in zip(first, projs):
        assert torch.equal(a["gq"], d["gq"]) and torch.equal(a["sgrad"], d["sgrad"]), "repeat differs"
    _oracle_check(projs, host, "split")


def test_layer_mixed_eligibility():
    """Projections the grouped kernels do not take (dW side 64 and 40, dX with
    the two-term scale, out = 40 < 512) mixed with ones they take."""
    shapes = [(512, 512), (64, 1024), (1024, 40), (256, 256), (136, 264)]
    projs, host = _make(1000, shapes, config_id=1603)
    ref = _single(projs)
    _layer(projs)
    _compare(projs, ref, "mixed")
    _oracle_check(projs, host, "mixed")


def test_layer_fp32_and_shared_input():
    shapes = [(264, 136), (264, 200), (264, 64)]
    projs, host = _make(300, shapes, act="f32", config_id=1604, shared_x=True)
    ref = _single(projs)
    _layer(projs)
    _compare(projs, ref, "fp32", dw_bitwise=True)   # fp32 runs the single-projection path
    _oracle_check(projs, host, "fp32")
    projs, host = _make(2048, [(1024, 1024)] * 3, config_id=1605, shared_x=True)   # q / k / v
    ref = _single(projs)
    _layer(projs)
    _compare(projs, ref, "qkv")


def test_layer_empty_projection():
    """An in = 0 projection: Y is the empty sum (0), sgrad 0; the others as usual."""
    projs, host = _make(512, [(512, 512), (512, 256)], config_id=1606)
    ni, no = 0, 64
    projs.append(dict(n_in=ni, n_out=no, q=torch.empty((0, no), dtype=torch.int8, device="cuda"),
                      scale=torch.ones(no, device="cuda"),
                      X=torch.empty((512, 0), dtype=torch.bfloat16, device="cuda"),
                      dY=torch.randn((512, no), device="cuda").bfloat16(), packed=tl.empty_packed(ni, no),
                      Y=torch.full((512, no), 7.0, device="cuda"), dX=torch.empty((512, 0), device="cuda"),
                      gq=torch.empty((0, no), device="cuda"), sgrad=torch.full((no,), 7.0, device="cuda")))
    ref = _single(projs[:2])
    _layer(projs)
    _compare(projs[:2], ref, "with empty")
    assert bool((projs[2]["Y"] == 0).all()) and bool((projs[2]["sgrad"] == 0).all())


def test_layer_class_walk_mid_block():
    """d = 1024, ffn 4096, 8192 tokens: four 1024 x 1024, 1024 -> 4096 and
    4096 -> 1024.  The forward's 128 items of 4096-long reductions and 1024
    of 1024 (dX the same) take the class-balanced walk."""
    shapes = [(1024, 1024)] * 4 + [(1024, 4096), (4096, 1024)]
    projs, host = _make(8192, shapes, config_id=1607)
    ref = _single(projs)
    _layer(projs)
    _compare(projs, ref, "mid block")
    _oracle_check(projs, host, "mid block", rows=12, cols=8)
    log("  layer mid block (class walk): equal to the single calls, oracle gate met")


def test_layer_bf16_y():
    """bf16 Y through the layer call (its own kernel instantiation, 2-byte
    stores from the transposed accumulators) equals the single-projection
    bf16 Y bit for bit, and the round-to-nearest-even of the fp32 Y."""
    shapes = [(1032, 520), (520, 1032), (256, 256)]
    projs, host = _make(1000, shapes, config_id=1608)
    tl.tern_layer_materialize(projs, 2)
    for d in projs:
        d["Y"] = torch.empty((1000, d["n_out"]), dtype=torch.bfloat16, device="cuda")
    tl.tern_layer_fwd(projs)
    torch.cuda.synchronize()
    for i, d in enumerate(projs):
        yb = torch.empty_like(d["Y"])
        tl.tern_linear_fwd(d["X"], d["packed"], d["scale"], yb)
        yf = torch.empty((1000, d["n_out"]), device="cuda")
        tl.tern_linear_fwd(d["X"], d["packed"], d["scale"], yf)
        torch.cuda.synchronize()
        assert torch.equal(d["Y"], yb), f"[{i}] layer bf16 Y differs from tern_linear_fwd"
        assert torch.equal(d["Y"], yf.to(torch.bfloat16)), f"[{i}] bf16 Y is not the RNE of the fp32 Y"
