"""The scale step (tern_scale_adamw through the C ABI) on the GPU against the
oracle's AdamW: fp32 on the device against f64, rel-L2 within the fp32 gate,
step by step (the oracle fed the device's state) and over several free-running
steps, and chained after the device's own scale gradient."""
import numpy as np
import pytest
import torch

import oracle
import synth
import ternary_weight_linear_tern_amd as tl
from gpu_util import DeviceProjection, TOL_F32, log, rel_l2

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


@pytest.mark.parametrize("out,lr,scale_lr,wd", [(4104, 2e-3, 1e-2, 0.0), (8, 1e-3, 1e-3, 0.1), (1000, 5e-4, 2e-3, 0.01)])
def test_scale_adamw_matches_oracle(o, out, lr, scale_lr, wd):
    log(f"scale AdamW out={out} lr={lr} scale_lr={scale_lr} wd={wd}")
    # the hyper-parameters are fp32 values on the device (the page declares
    # them float); the oracle gets those same values (1 - float(0.999) differs
    # from 1 - 0.999 by 1.3e-5 relative)
    f32 = lambda x: float(np.float32(x))
    lr, scale_lr, wd = f32(lr), f32(scale_lr), f32(wd)
    hp = dict(b1=f32(0.9), b2=f32(0.999), eps=f32(1e-8), wd=wd)
    rng = np.random.default_rng(out)
    s0 = rng.uniform(0.01, 0.1, out).astype(np.float32)
    sc = torch.from_numpy(s0).cuda()
    m = torch.zeros(out, device="cuda")
    v = torch.zeros(out, device="cuda")
    free = (s0.astype(np.float64), np.zeros(out), np.zeros(out))
    for t in range(1, 7):
        g = rng.normal(0.0, 1e-2, out).astype(np.float32)
        g[:: 17] = 0.0
        before = (sc.cpu().numpy().astype(np.float64), m.cpu().numpy().astype(np.float64),
                  v.cpu().numpy().astype(np.float64))
        tl.tern_scale_adamw(torch.from_numpy(g).cuda(), sc, m, v, t, lr, scale_lr, wd=wd)
        torch.cuda.synchronize()
        got = (sc.cpu().numpy(), m.cpu().numpy(), v.cpu().numpy())
        want = o.scale_adamw(g, *before, t, lr, scale_lr, **hp)
        free = o.scale_adamw(g, *free, t, lr, scale_lr, **hp)
        for name, a, b, c in zip(("scale", "m", "v"), got, want, free):
            e1, e2 = rel_l2(a, b), rel_l2(a, c)
            assert e1 <= TOL_F32 and e2 <= TOL_F32, f"step {t} {name}: relL2 {e1:.2e} / {e2:.2e}"
        # the step itself, not only the (much larger) scale, meets the gate
        assert rel_l2(got[0] - before[0], want[0] - before[0]) <= 1e-4, f"step {t}: scale increment"


def test_scale_adamw_after_backward(o):
    """sgrad from tern_linear_bwd_dw, then the scale step: the new scale meets
    the gate against the oracle's sgrad followed by the oracle's AdamW."""
    p = synth.make_inputs(512, 264, 520, act="bf16", config_id=880)
    d = DeviceProjection(p)
    d.materialize()
    tl.tern_linear_bwd_dw(d.X, d.dY, d.packed, d.scale, d.gq, d.sgrad, d.ws)
    m = torch.zeros_like(d.sgrad)
    v = torch.zeros_like(d.sgrad)
    new_scale = d.scale.clone()
    tl.tern_scale_adamw(d.sgrad, new_scale, m, v, 1, 1e-3, 1e-3)
    torch.cuda.synchronize()
    _, _, sgo = o.linear_wgrad(p.X, p.dY, p.q, p.theta, p.scale)
    f32 = lambda x: float(np.float32(x))
    want, _, _ = o.scale_adamw(sgo, p.scale.astype(np.float64), np.zeros(520), np.zeros(520), 1, f32(1e-3),
                               f32(1e-3), f32(0.9), f32(0.999), f32(1e-8), 0.0)
    got = new_scale.cpu().numpy()
    # the first AdamW step is lr * sign(g) (up to eps), so the device's sgrad
    # rounding can only matter where |sgrad| is tiny; the new scales agree
    e = rel_l2(got - p.scale, want - p.scale)
    log(f"  scale step after backward: relL2 of the step {e:.2e}")
    assert e <= 2e-3
