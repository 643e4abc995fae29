"""Many repetitions of the layer step stay bitwise equal, through the C ABI on the GPU.

The forward / dX kernel orders each wave's own loads and stores by vmcnt
arithmetic and has one workgroup barrier per chunk, after which a wave reads
the half of the shared activation stage that its partner loaded; the
accumulating dX keeps a private ring and no barrier; the dW kernel's refill
runs ahead of a barrier.  A wait that came up short would read a stage before
its data landed and change some outputs from one run to the next.  Every output
is deterministic (fixed tiles, fixed summation orders), so the step is
repeated, eagerly and as one graph replay, with the outputs filled with NaN
before every repetition, and each repetition must equal the first bit for bit.
"""
import numpy as np
import pytest
import torch

import synth
import ternary_weight_linear_tern_amd as tl
from gpu_util import log, to_dev

pytestmark = pytest.mark.gpu

KEYS = ("Y", "dX", "gq", "sgrad")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    tl.lib()
    yield
    torch.cuda.synchronize()


def _workload(name):
    w = synth.WORKLOADS[name]
    projs = []
    for i, (_, ni, no) in enumerate(w.projs):
        p = synth.workload_inputs(w, i)
        projs.append(dict(n_in=ni, n_out=no, X=to_dev(p.X), dY=to_dev(p.dY), q=to_dev(p.q), scale=to_dev(p.scale),
                          packed=tl.empty_packed(ni, no), Y=torch.empty((w.T, no), device="cuda"),
                          dX=torch.empty((w.T, ni), device="cuda"), gq=torch.empty((ni, no), device="cuda"),
                          sgrad=torch.empty((no,), device="cuda")))
    ws = tl.empty_layer_workspace([(d["n_in"], d["n_out"]) for d in projs], w.T)
    return w, projs, ws


@pytest.mark.parametrize("name,reps,graph", [("mid", 100, False), ("rwkv_small", 200, True), ("large", 30, True)])
def test_repeated_step_bitwise(name, reps, graph):
    w, projs, ws = _workload(name)
    log(f"{name}: {reps} {'graph replays' if graph else 'eager steps'}")

    def step():
        tl.tern_layer_materialize(projs, w.theta)
        tl.tern_layer_fwd(projs)
        tl.tern_layer_bwd_dx(projs)
        tl.tern_layer_bwd_dw(projs, ws)

    step()
    torch.cuda.synchronize()
    ref = [{k: d[k].clone() for k in KEYS} for d in projs]
    g, s = None, torch.cuda.current_stream()
    if graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        tl.tern_graph_begin(s)
        with torch.cuda.stream(s):
            step()
        g = tl.tern_graph_end(s)
    try:
        for k in range(reps):
            with torch.cuda.stream(s):
                for d in projs:
                    for key in KEYS:
                        d[key].fill_(float("nan"))
                if graph:
                    tl.tern_graph_launch(g, s)
                else:
                    step()
            s.synchronize()
            for i, d in enumerate(projs):
                for key in KEYS:
                    assert torch.equal(d[key], ref[i][key]), f"{name}: repetition {k}, projection {i}: {key} changed"
    finally:
        if g is not None:
            tl.tern_graph_destroy(g)
    assert all(bool(torch.isfinite(d[k]).all()) for d in projs for k in KEYS)
