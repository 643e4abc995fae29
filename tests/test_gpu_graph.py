"""Graphs of library calls on the GPU (tern_graph_* through the C ABI).

One recording of materialize + forward + backward for two projections of
different shapes is replayed several times.  Between replays the program does
eager work of its own (fills the outputs with NaN, replaces inputs in place,
synchronises); every replay must reproduce, bit for bit, what the eager calls
give on the inputs the buffers hold at that time, and one replay is also held
to the oracle's gate.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import ternary_weight_linear_tern_amd as tl
from gpu_util import DeviceProjection, log, rel_l2, tol_for

pytestmark = pytest.mark.gpu

SHAPES = [(1000, 264, 520), (777, 136, 1032)]   # T, in, out (bf16 activations)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    tl.lib()
    yield
    torch.cuda.synchronize()


def _record(projs, s):
    for d in projs:
        tl.tern_materialize(d.q, d.p.theta, d.packed, s)
        tl.tern_linear_fwd(d.X, d.packed, d.scale, d.Y, s)
        tl.tern_linear_bwd(d.X, d.dY, d.packed, d.scale, d.dX, d.gq, d.sgrad, d.ws, s)


def _outputs(projs):
    torch.cuda.synchronize()
    return [{k: getattr(d, k).clone() for k in ("packed", "Y", "dX", "gq", "sgrad")} for d in projs]


def _poison(projs, s):
    with torch.cuda.stream(s):
        for d in projs:
            for t in (d.Y, d.dX, d.gq, d.sgrad):
                t.fill_(float("nan"))
            d.packed.fill_(-1)


def _same(got, want, tag):
    for j, (g, w) in enumerate(zip(got, want)):
        for k in w:
            assert torch.equal(g[k], w[k]), f"{tag}: projection {j} {k} differs from the eager result"


def test_graph_replays_match_eager():
    ps = [synth.make_inputs(T, i, o, act="bf16", config_id=700 + n) for n, (T, i, o) in enumerate(SHAPES)]
    projs = [DeviceProjection(p) for p in ps]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())

    log("graph: eager reference")
    _record(projs, s)              # eager: runs now
    eager = _outputs(projs)

    log("graph: recording")
    tl.tern_graph_begin(s)
    try:
        _record(projs, s)          # recorded: nothing runs
    finally:
        g = tl.tern_graph_end(s)
    assert g.value, "no graph handle"
    try:
        for rep in range(3):
            log(f"graph: replay {rep}")
            _poison(projs, s)
            s.synchronize()
            tl.tern_graph_launch(g, s)
            s.synchronize()
            _same(_outputs(projs), eager, f"replay {rep}")

        # new input contents in the same buffers: the replay reads them
        log("graph: replay on replaced inputs")
        ps2 = [synth.make_inputs(T, i, o, act="bf16", config_id=710 + n) for n, (T, i, o) in enumerate(SHAPES)]
        fresh = [DeviceProjection(p) for p in ps2]
        for d, f in zip(projs, fresh):
            for k in ("X", "dY", "q", "scale"):
                getattr(d, k).copy_(getattr(f, k))
        torch.cuda.synchronize()
        _poison(projs, s)
        tl.tern_graph_launch(g, s)
        tl.tern_graph_launch(g, s)   # two replays back to back give the same result
        replayed = _outputs(projs)
        for d, f in zip(fresh, ps2):
            d.step()
        _same(replayed, _outputs(fresh), "replay on replaced inputs")
    finally:
        tl.tern_graph_destroy(g)

    # the replayed results also meet the oracle's gate
    o = oracle.get()
    p, r = ps2[0], replayed[0]
    tol = tol_for(p.act)
    Yo = o.linear_fwd(p.X, p.q, p.theta, p.scale)
    dXo = o.linear_dx(p.dY, p.q, p.theta, p.scale)
    _, gqo, sgo = o.linear_wgrad(p.X, p.dY, p.q, p.theta, p.scale)
    n_in, n_out = p.q.shape
    pk = tl.packed_canonical(r["packed"], n_in, n_out).cpu().numpy().view(np.uint32)
    assert np.array_equal(pk, o.pack(o.tern(p.q, p.theta))), "replayed packing differs from the oracle"
    errs = dict(Y=rel_l2(r["Y"].cpu().numpy(), Yo), dX=rel_l2(r["dX"].cpu().numpy(), dXo),
                gq=rel_l2(r["gq"].cpu().numpy(), gqo), sgrad=rel_l2(r["sgrad"].cpu().numpy(), sgo))
    log(f"graph replay relL2 {errs}")
    for k, e in errs.items():
        assert e <= tol, f"replayed {k} relL2 {e:.3e} > {tol:.1e}"


def test_graph_invalid_call_records_nothing():
    """While recording, a call with bad arguments is refused by its checks
    before any HIP call, so the recording stays valid and replays only the
    valid calls."""
    p = synth.make_inputs(64, 64, 64, act="bf16", config_id=720)
    d = DeviceProjection(p)
    s = torch.cuda.Stream()
    d.materialize()
    torch.cuda.synchronize()
    bad = torch.empty((64, 60), dtype=torch.float32, device="cuda")   # Y with the wrong width
    tl.tern_graph_begin(s)
    try:
        with pytest.raises(tl.TernError):
            tl.tern_linear_fwd(d.X, d.packed, d.scale[:60], bad, s)
        tl.tern_linear_fwd(d.X, d.packed, d.scale, d.Y, s)
    finally:
        g = tl.tern_graph_end(s)
    try:
        bad.fill_(7.0)
        d.Y.fill_(float("nan"))
        torch.cuda.synchronize()
        tl.tern_graph_launch(g, s)
        s.synchronize()
        Y1 = d.Y.clone()
        d.fwd()
        torch.cuda.synchronize()
        assert torch.equal(Y1, d.Y), "replay differs from the eager forward"
        assert bool((bad == 7.0).all()), "the refused call wrote its output"
    finally:
        tl.tern_graph_destroy(g)


@pytest.mark.parametrize("layout", ["products", "projections"])
def test_graph_branches_match_eager(layout):
    """A recording on three streams replays to the eager results bit for bit:
    products (forward on the first stream, dX and dW on branches that fork
    after each materialize) or projections (each projection's whole chain on
    one of the streams); the branches rejoin the first stream at the end."""
    ps = [synth.make_inputs(T, i, o, act="bf16", config_id=730 + n) for n, (T, i, o) in enumerate(SHAPES)]
    projs = [DeviceProjection(p) for p in ps]
    for d in projs:
        d.step()
    eager = _outputs(projs)
    s0, s1, s2 = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()

    def fork(src, dst):
        e = torch.cuda.Event()
        e.record(src)
        dst.wait_event(e)

    tl.tern_graph_begin(s0)
    try:
        fork(s0, s1)
        fork(s0, s2)
        for j, d in enumerate(projs):
            if layout == "products":
                tl.tern_materialize(d.q, d.p.theta, d.packed, s0)
                fork(s0, s1)
                fork(s0, s2)
                tl.tern_linear_fwd(d.X, d.packed, d.scale, d.Y, s0)
                tl.tern_linear_bwd_dx(d.dY, d.packed, d.scale, d.dX, stream=s1)
                tl.tern_linear_bwd_dw(d.X, d.dY, d.packed, d.scale, d.gq, d.sgrad, d.ws, s2)
            else:
                st = (s0, s1, s2)[j % 3]
                tl.tern_materialize(d.q, d.p.theta, d.packed, st)
                tl.tern_linear_fwd(d.X, d.packed, d.scale, d.Y, st)
                tl.tern_linear_bwd_dx(d.dY, d.packed, d.scale, d.dX, stream=st)
                tl.tern_linear_bwd_dw(d.X, d.dY, d.packed, d.scale, d.gq, d.sgrad, d.ws, st)
        fork(s1, s0)
        fork(s2, s0)
    finally:
        g = tl.tern_graph_end(s0)
    try:
        for rep in range(3):
            log(f"graph branches ({layout}): replay {rep}")
            _poison(projs, s0)
            s0.synchronize()
            tl.tern_graph_launch(g, s0)
            s0.synchronize()
            _same(_outputs(projs), eager, f"branched ({layout}) replay {rep}")
    finally:
        tl.tern_graph_destroy(g)
