"""A seeded sweep of random shapes and input laws against the oracle, through
the C ABI on the GPU.

The fixed shape lists of the other parity tests are chosen by hand; this sweep
draws 24 problems from one seed: T in [1, 900], in and out multiples of 8 in
[8, 632], bf16 or fp32 activations, theta in {1, 2, 3, 5, 7}, uniform or
skewed q, uniform or lognormal scales (the laws of the benchmark configs), and
a bf16 Y on some bf16 problems.  Each is materialised, run forward and
backward, and compared with the oracle: the handle bit for bit, every output
within the gate, and every fp32 output within its per-element rounding bound.
Sizes that no hand-picked list contains (tiny T, one 8-wide tile, K not a
multiple of any chunk) land on every kernel path: the persistent kernels,
the smaller tiles, the two-term dX scale and the fp32 kernels.
Then the problems with equal T go through the layer calls as well, and eight
larger random ragged shapes run the persistent kernels, compared on sampled
rows and columns.
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


def _cases(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        T = int(rng.integers(1, 901))
        n_in, n_out = 8 * int(rng.integers(1, 80)), 8 * int(rng.integers(1, 80))
        act = "bf16" if rng.random() < 0.75 else "f32"
        theta = int(rng.choice([1, 2, 3, 5, 7]))
        q_law = "skewed" if rng.random() < 0.3 else "uniform"
        scale_law = "lognormal" if rng.random() < 0.3 else "uniform"
        y_bf16 = act == "bf16" and rng.random() < 0.3
        out.append((k, T, n_in, n_out, act, theta, q_law, scale_law, y_bf16))
    return out


CASES = _cases()


def _inputs(case):
    k, T, n_in, n_out, act, theta, q_law, scale_law, _ = case
    return synth.make_inputs(T, n_in, n_out, act=act, q_law=q_law, scale_law=scale_law, theta=theta,
                             config_id=2100 + k)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}x{c[3]}-{c[4]}-t{c[5]}")
def test_sweep_single(o, case):
    k, T, n_in, n_out, act, theta, q_law, scale_law, y_bf16 = case
    log(f"sweep {k}: T={T} in={n_in} out={n_out} {act} theta={theta} {q_law} {scale_law} y_bf16={y_bf16}")
    p = _inputs(case)
    d = DeviceProjection(p, y_bf16=y_bf16)
    d.step()
    r = d.results()
    assert np.array_equal(r["packed"], o.pack(o.tern(p.q, p.theta))), "packing differs from the oracle"
    want = {"Y": o.linear_fwd(p.X, p.q, p.theta, p.scale), "dX": o.linear_dx(p.dY, p.q, p.theta, p.scale)}
    _, want["gq"], want["sgrad"] = o.linear_wgrad(p.X, p.dY, p.q, p.theta, p.scale)
    tol = tol_for(act)
    for key in ("Y", "dX", "gq", "sgrad"):
        e = rel_l2(r[key], want[key])
        assert e <= tol, f"{key} relL2 {e:.3e} above {tol:.0e}"
    exact = {key: r[key] for key in ("dX", "gq", "sgrad")}
    if not y_bf16:
        exact["Y"] = r["Y"]
    check_elements(o, p, exact, want, tag=f"sweep {k}")


def _big_cases(n=8, seed=2025):
    rng = np.random.default_rng(seed)
    return [(k, int(rng.integers(256, 4097)), 8 * int(rng.integers(32, 257)), 8 * int(rng.integers(32, 257)),
             "lognormal" if rng.random() < 0.5 else "uniform") for k in range(n)]


@pytest.mark.parametrize("case", _big_cases(), ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}x{c[3]}")
def test_sweep_large_sampled(o, case):
    """Random ragged shapes large enough for the persistent kernels
    (T up to 4096, in and out up to 2048, bf16), compared on sampled rows of
    Y and dX and sampled columns of gq and sgrad, each sampled element within
    its rounding bound."""
    k, T, n_in, n_out, scale_law = case
    log(f"large sweep {k}: T={T} in={n_in} out={n_out} {scale_law}")
    p = synth.make_inputs(T, n_in, n_out, act="bf16", scale_law=scale_law, config_id=2300 + k)
    d = DeviceProjection(p)
    d.step()
    r = d.results()
    assert np.array_equal(r["packed"], o.pack(o.tern(p.q, p.theta))), "packing differs from the oracle"
    rows = synth.sample_indices(2400 + k, 24, T)
    cols = synth.sample_indices(2500 + k, 12, n_out)
    want = {"Y": o.linear_fwd(p.X, p.q, p.theta, p.scale, rows=rows),
            "dX": o.linear_dx(p.dY, p.q, p.theta, p.scale, rows=rows)}
    _, gq, sg = o.linear_wgrad(p.X, p.dY, p.q, p.theta, p.scale, cols=cols)
    got = {"Y": r["Y"][rows], "dX": r["dX"][rows]}
    for key in ("Y", "dX"):
        e = rel_l2(got[key], want[key])
        assert e <= 2e-3, f"{key} relL2 {e:.3e} on sampled rows"
    for key, g, w in (("gq", r["gq"][:, cols], gq), ("sgrad", r["sgrad"][cols], sg)):
        e = rel_l2(g, w)
        assert e <= 2e-3, f"{key} relL2 {e:.3e} on sampled columns"
    check_elements(o, p, got, want, rows=rows, tag=f"large sweep {k}")
    check_elements(o, p, {"gq": r["gq"][:, cols], "sgrad": r["sgrad"][cols]}, {"gq": gq, "sgrad": sg}, cols=cols,
                   tag=f"large sweep {k} dW")


def test_sweep_layer(o):
    """The bf16 problems of the sweep, regrouped to one T per layer (the first
    problem's T of each group of three), through the layer calls."""
    bf = [c for c in CASES if c[4] == "bf16"]
    groups = [bf[i:i + 3] for i in range(0, len(bf), 3)]
    for gi, g in enumerate(groups):
        T = g[0][1]
        projs, host = [], []
        for c in g:
            k, _, n_in, n_out, act, theta, q_law, scale_law, _ = c
            p = synth.make_inputs(T, n_in, n_out, act="bf16", q_law=q_law, scale_law=scale_law, theta=2,
                                  config_id=2200 + k)
            projs.append(dict(n_in=n_in, n_out=n_out, q=to_dev(p.q), scale=to_dev(p.scale), X=to_dev(p.X),
                              dY=to_dev(p.dY), packed=tl.empty_packed(n_in, n_out),
                              Y=torch.empty((T, n_out), device="cuda"), dX=torch.empty((T, n_in), device="cuda"),
                              gq=torch.empty((n_in, n_out), device="cuda"), sgrad=torch.empty((n_out,), device="cuda")))
            host.append(p)
        log(f"sweep layer {gi}: T={T} {[(d['n_in'], d['n_out']) for d in projs]}")
        ws = tl.empty_layer_workspace([(d["n_in"], d["n_out"]) for d in projs], T)
        tl.tern_layer_materialize(projs, 2)
        tl.tern_layer_fwd(projs)
        tl.tern_layer_bwd_dx(projs)
        tl.tern_layer_bwd_dw(projs, ws)
        torch.cuda.synchronize()
        for i, (d, p) in enumerate(zip(projs, host)):
            got = {key: d[key].cpu().numpy() for key in ("Y", "dX", "gq", "sgrad")}
            want = {"Y": o.linear_fwd(p.X, p.q, p.theta, p.scale), "dX": o.linear_dx(p.dY, p.q, p.theta, p.scale)}
            _, want["gq"], want["sgrad"] = o.linear_wgrad(p.X, p.dY, p.q, p.theta, p.scale)
            for key in got:
                e = rel_l2(got[key], want[key])
                assert e <= 2e-3, f"layer {gi} projection {i}: {key} relL2 {e:.3e}"
            check_elements(o, p, got, want, tag=f"sweep layer {gi} projection {i}")
