"""Both tile shapes of the persistent forward / dX kernel, through the C ABI.

The launch takes 512 x 128 tiles (output columns x tokens) unless their column
padding adds more than 3 % of multiply-adds over 256 x 256 tiles; then, and
for the accumulating dX, it takes 256 x 256 tiles (the choice itself is pinned
on the CPU by the planner check).  Each layer here lands on one shape for both
products: columns on the 512 grid (wide), or 768 and 1032 columns (square).
Every output is compared with the oracle element by element (rel-L2 gate and
each element within its rounding bound), the bf16 Y with the round-to-nearest-
even of the fp32 Y bit for bit, and the two shapes with each other on one
projection they share.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import ternary_weight_linear_tern_amd as tl
from gpu_util import check_elements, log, rel_l2, to_dev

pytestmark = pytest.mark.gpu

T = 1000   # 7 full 128-token tiles and a ragged one; 3 full 256-token tiles and a ragged one


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


def _layer(shapes, config_id, proj_ids=None):
    projs, host = [], []
    for i, (ni, no) in enumerate(shapes):
        p = synth.make_inputs(T, ni, no, act="bf16", config_id=config_id,
                              proj_id=i if proj_ids is None else proj_ids[i])
        projs.append(dict(n_in=ni, n_out=no, q=to_dev(p.q), scale=to_dev(p.scale), X=to_dev(p.X), dY=to_dev(p.dY),
                          packed=tl.empty_packed(ni, no), Y=torch.empty((T, no), device="cuda"),
                          dX=torch.empty((T, ni), device="cuda"), gq=torch.empty((ni, no), device="cuda"),
                          sgrad=torch.empty((no,), device="cuda")))
        host.append(p)
    ws = tl.empty_layer_workspace(shapes, T)
    tl.tern_layer_materialize(projs, 2)
    tl.tern_layer_fwd(projs)
    tl.tern_layer_bwd_dx(projs)
    tl.tern_layer_bwd_dw(projs, ws)
    # the bf16 Y of the same kernels
    ybf = [torch.empty((T, d["n_out"]), dtype=torch.bfloat16, device="cuda") for d in projs]
    tl.tern_layer_fwd([dict(d, Y=y) for d, y in zip(projs, ybf)])
    torch.cuda.synchronize()
    return projs, host, ybf


# (in, out) per projection: forward columns = out, dX columns = in
SHAPES = {
    "wide": [(1024, 512), (512, 1536), (2048, 1024)],
    "square": [(768, 1032), (1032, 768), (512, 1024)],
}


@pytest.mark.parametrize("kind", ["wide", "square"])
def test_tile_shape_against_oracle(o, kind):
    shapes = SHAPES[kind]
    log(f"{kind} tiles: T={T} {shapes}")
    projs, host, ybf = _layer(shapes, 2600 + (kind == "square"))
    for i, (d, p) in enumerate(zip(projs, host)):
        got = {k: d[k].cpu().numpy() for k in ("Y", "dX", "gq", "sgrad")}
        want = {"Y": o.linear_fwd(p.X, p.q, p.theta, p.scale), "dX": o.linear_dx(p.dY, p.q, p.theta, p.scale)}
        _, want["gq"], want["sgrad"] = o.linear_wgrad(p.X, p.dY, p.q, p.theta, p.scale)
        for k in got:
            e = rel_l2(got[k], want[k])
            assert e <= 2e-3, f"{kind} projection {i}: {k} relL2 {e:.3e}"
        check_elements(o, p, got, want, tag=f"{kind} tiles, projection {i}")
        yb = ybf[i].float().cpu().numpy()
        ref = torch.from_numpy(got["Y"]).bfloat16().float().numpy()
        assert np.array_equal(yb, ref), f"{kind} projection {i}: bf16 Y is not the rounded fp32 Y"


def test_tile_shapes_agree():
    """The (512, 1024) projection runs on square tiles in one layer and on wide
    tiles in another: every output is bit for bit the same (the same sums in
    the same order along K, whatever the tile)."""
    log("one projection on both tile shapes")
    a, _, _ = _layer(SHAPES["square"], 2601)
    b, _, _ = _layer([SHAPES["square"][2]] + SHAPES["wide"][:1], 2601, proj_ids=[2, 5])
    for k in ("Y", "dX", "gq", "sgrad"):
        x, y = a[2][k], b[0][k]
        if k in ("gq", "sgrad"):
            # dW's split over tokens is planned per layer: fp32 rounding apart
            e = rel_l2(y.cpu().numpy(), x.cpu().numpy().astype(np.float64))
            assert e <= 1e-6, f"{k} differs by relL2 {e:.3e}"
        else:
            assert torch.equal(x, y), f"{k} differs between the tile shapes"
