"""Calls on two streams at once, through the C ABI on the GPU.

The library keeps no state between calls (every buffer is the caller's, the
plans are computed on the host per call), so independent projections enqueued
on two streams that run concurrently must give exactly the results of the same
calls run one after the other: the same kernels, tiles and summation orders.
Checked for the single-projection calls (materialize, forward, backward with
its own workspace each) and for two layers through the layer calls.
"""
import numpy as np
import pytest
import torch

import synth
import ternary_weight_linear_tern_amd as tl
from gpu_util import DeviceProjection, log, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    tl.lib()
    yield
    torch.cuda.synchronize()


def _same(a, b, tag):
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=True), f"{tag}: {k} differs between streams and sequence"


def test_single_calls_on_two_streams():
    shapes = [(2056, 1032, 1032), (1000, 2056, 520)]
    ds = [DeviceProjection(synth.make_inputs(T, i, o, act="bf16", config_id=2001 + j))
          for j, (T, i, o) in enumerate(shapes)]
    log("single calls, sequence then two streams")
    for d in ds:
        d.step()
    seq = [d.results() for d in ds]
    for d in ds:   # overwrite the outputs so that stale values cannot pass
        for t in (d.Y, d.dX, d.gq, d.sgrad):
            t.fill_(float("nan"))
    cur = torch.cuda.current_stream()
    streams = [torch.cuda.Stream() for _ in ds]
    for s in streams:
        s.wait_stream(cur)
    for d, s in zip(ds, streams):
        with torch.cuda.stream(s):
            d.step()
    for s in streams:
        cur.wait_stream(s)
    torch.cuda.synchronize()
    for j, d in enumerate(ds):
        _same(seq[j], d.results(), f"projection {j}")


def _layer_buffers(T, shapes, config_id):
    projs = []
    for i, (ni, no) in enumerate(shapes):
        p = synth.make_inputs(T, ni, no, act="bf16", config_id=config_id, proj_id=i)
        projs.append(dict(n_in=ni, n_out=no, q=to_dev(p.q), scale=to_dev(p.scale), X=to_dev(p.X), dY=to_dev(p.dY),
                          packed=tl.empty_packed(ni, no), Y=torch.empty((T, no), device="cuda"),
                          dX=torch.empty((T, ni), device="cuda"), gq=torch.empty((ni, no), device="cuda"),
                          sgrad=torch.empty((no,), device="cuda")))
    return projs, tl.empty_layer_workspace(shapes, T)


def _layer_step(projs, ws):
    tl.tern_layer_materialize(projs, 2)
    tl.tern_layer_fwd(projs)
    tl.tern_layer_bwd_dx(projs)
    tl.tern_layer_bwd_dw(projs, ws)


def _layer_results(projs):
    torch.cuda.synchronize()
    return [{k: d[k].cpu().numpy() for k in ("Y", "dX", "gq", "sgrad")} for d in projs]


def test_layer_calls_on_two_streams():
    layers = [_layer_buffers(2048, [(512, 512), (512, 2048), (2048, 512)], 2011),
              _layer_buffers(4096, [(1024, 1024), (1024, 1024)], 2012)]
    log("layer calls, sequence then two streams")
    for projs, ws in layers:
        _layer_step(projs, ws)
    seq = [_layer_results(projs) for projs, _ in layers]
    for projs, _ in layers:
        for d in projs:
            for k in ("Y", "dX", "gq", "sgrad"):
                d[k].fill_(float("nan"))
    cur = torch.cuda.current_stream()
    streams = [torch.cuda.Stream() for _ in layers]
    for s in streams:
        s.wait_stream(cur)
    for (projs, ws), s in zip(layers, streams):
        with torch.cuda.stream(s):
            _layer_step(projs, ws)
    for s in streams:
        cur.wait_stream(s)
    for j, (projs, _) in enumerate(layers):
        got = _layer_results(projs)
        for i, (a, b) in enumerate(zip(seq[j], got)):
            _same(a, b, f"layer {j} projection {i}")
