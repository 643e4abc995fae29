"""Invariants of the method checked through the kernels (C ABI, on the GPU).

* All-zero ternary matrix (theta above every |q|): W_eff = 0, so Y, dX and
  sgrad are exactly zero, while gq = G * scale still carries the weight
  gradient (page "train_gpu.cu", tg_tern_from_q's dead zone; tg_gq, tg_scale_grad).
* Sign matrix: scale = 1 (the trainer's initial scale) and every |q| >= theta
  make W_eff a +-1 matrix.  With activations in {-1, 0, 1} every product and
  every partial sum is a small integer, exact in fp32 whatever the summation
  order, so the device results equal the oracle's f64 results bit for bit.
* A non-finite activation in token row t + 1 leaves row t of Y (and of dX)
  untouched: the kernels read no activation bytes past the reduction length.
* A NaN scale poisons its own columns of Y and gq and, in dX, what each path's
  operand makes of NaN * tern (see test_nonfinite_scale).

Shapes are chosen so that all three products run the persistent
kernels (ragged in every dimension, the dW product split over tokens) and, for
comparison, the fp32 path.
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


def _small_int_act(seed, shape, act):
    """Activations in {-1, 0, 1} (exact in bf16 and fp32)."""
    rng = np.random.default_rng(seed)
    a = rng.integers(-1, 2, size=shape).astype(np.float32)
    return synth.to_bf16_bits(a) if act == "bf16" else a


@pytest.mark.parametrize("T,n_in,n_out,act", [(4000, 1032, 1032, "bf16"), (2056, 2056, 2056, "bf16"),
                                              (1000, 264, 136, "f32")])
def test_all_zero_tern(o, T, n_in, n_out, act):
    """theta = 8 > max |q| = 7: Y, dX, sgrad exactly 0; gq = G * scale."""
    log(f"all-zero tern {T}x{n_in}x{n_out} {act}")
    p = synth.make_inputs(T, n_in, n_out, act=act, config_id=1301)
    p.theta = 8
    d = DeviceProjection(p)
    d.step()
    r = d.results()
    assert not np.any(r["packed"]), "theta above every |q| must give the all-zero code"
    for k in ("Y", "dX", "sgrad"):
        assert np.all(r[k] == 0.0), f"{k} is not exactly zero with an all-zero ternary matrix"
    _, gq, sg = o.linear_wgrad(p.X, p.dY, p.q, p.theta, p.scale)
    assert np.all(sg == 0.0)
    e = rel_l2(r["gq"], gq)
    log(f"  gq relL2 {e:.3e}")
    assert e <= tol_for(act)
    check_elements(o, p, {"gq": r["gq"]}, {"gq": gq}, tag="all-zero tern gq")


@pytest.mark.parametrize("T,n_in,n_out,act", [(4000, 1032, 1032, "bf16"), (2056, 2056, 2056, "bf16"),
                                              (1000, 264, 136, "f32")])
def test_sign_matrix_bitwise(o, T, n_in, n_out, act):
    """scale = 1, |q| >= theta everywhere, activations in {-1, 0, 1}: the
    device equals the oracle bit for bit in Y, dX, gq and sgrad."""
    log(f"sign matrix {T}x{n_in}x{n_out} {act}")
    p = synth.make_inputs(T, n_in, n_out, act=act, config_id=1302)
    rng = np.random.default_rng(1302)
    mag = rng.integers(2, 8, size=(n_in, n_out))
    sign = rng.integers(0, 2, size=(n_in, n_out)) * 2 - 1
    p.q = (mag * sign).astype(np.int8)
    p.scale = np.ones(n_out, dtype=np.float32)
    p.X = _small_int_act(11, (T, n_in), act)
    p.dY = _small_int_act(12, (T, n_out), act)
    d = DeviceProjection(p)
    d.step()
    r = d.results()
    want_pk = o.pack(o.tern(p.q, p.theta))
    assert np.array_equal(r["packed"], want_pk)
    want = dict(Y=o.linear_fwd(p.X, p.q, p.theta, p.scale), dX=o.linear_dx(p.dY, p.q, p.theta, p.scale))
    _, want["gq"], want["sgrad"] = o.linear_wgrad(p.X, p.dY, p.q, p.theta, p.scale)
    for k in ("Y", "dX", "gq", "sgrad"):
        got = np.asarray(r[k], dtype=np.float64)
        bad = np.argwhere(got != want[k])
        assert bad.size == 0, f"{k} differs from the oracle at {tuple(bad[0])}: {got[tuple(bad[0])]} " \
                              f"vs {want[k][tuple(bad[0])]} ({bad.shape[0]} elements)"


def test_nonfinite_next_row_does_not_leak():
    """An Inf in X[t + 1, 0] (a NaN in dY[t + 1, 0]) changes only row t + 1
    of Y (of dX).  K = 1032 is not a multiple of the 32-wide chunk, so the
    last chunk and the padding chunk reach past the end of each row."""
    T, n_in, n_out = 4000, 1032, 1032
    log(f"non-finite next row {T}x{n_in}x{n_out}")
    p = synth.make_inputs(T, n_in, n_out, act="bf16", config_id=1303)
    d = DeviceProjection(p)
    d.materialize()
    d.fwd()
    tl.tern_linear_bwd_dx(d.dY, d.packed, d.scale, d.dX)
    torch.cuda.synchronize()
    Y0, dX0 = d.Y.clone(), d.dX.clone()
    rows = [0, 255, 1000, 1999, T - 2]   # no row is another's successor
    for t in rows:
        d.X[t + 1, 0] = float("inf")
        d.dY[t + 1, 0] = float("nan")
    d.fwd()
    tl.tern_linear_bwd_dx(d.dY, d.packed, d.scale, d.dX)
    torch.cuda.synchronize()
    hit = set(t + 1 for t in rows)
    assert not hit & set(rows)
    keep = torch.tensor([i for i in range(T) if i not in hit], device="cuda")
    assert torch.equal(d.Y[keep], Y0[keep]), "a non-finite X element changed another token row of Y"
    assert torch.equal(d.dX[keep], dX0[keep]), "a non-finite dY element changed another token row of dX"
    for t in rows:
        assert bool(torch.isfinite(d.Y[t]).all()) and bool(torch.isfinite(d.dX[t]).all())


@pytest.mark.parametrize("T,n_in,n_out,act", [(1000, 1032, 1032, "bf16"), (300, 264, 136, "f32")])
def test_nonfinite_scale(o, T, n_in, n_out, act):
    """A NaN scale[c]: the forward multiplies column c's sums by it, so Y[:, c]
    and gq[:, c] are NaN and every other column is unchanged; sgrad does not
    involve the scale.  dX: the fp32 path multiplies the decoded code by the
    scale, so W_eff[:, c] = NaN * tern is NaN even where the code is 0 and every
    dX entry is NaN, as in the oracle; the bf16 persistent kernel builds its
    operand as +-bf16(scale) selected by the code (a zero code gives an exact
    0, NaN * 0 is never formed), so dX[t, r] is NaN where tern[r, c] != 0 and
    bitwise unchanged where it is 0.  Non-finite inputs have no parity gate;
    this pins what each path does."""
    log(f"non-finite scale {T}x{n_in}x{n_out} {act}")
    p = synth.make_inputs(T, n_in, n_out, act=act, config_id=1304)
    d = DeviceProjection(p)
    d.step()
    r0 = d.results()
    c = 37
    d.scale[c] = float("nan")
    d.step()
    r = d.results()
    other = [j for j in range(n_out) if j != c]
    assert np.all(np.isnan(r["Y"][:, c])) and np.array_equal(r["Y"][:, other], r0["Y"][:, other])
    assert np.all(np.isnan(r["gq"][:, c])) and np.array_equal(r["gq"][:, other], r0["gq"][:, other])
    assert np.array_equal(r["sgrad"], r0["sgrad"]), "sgrad does not involve the scale"
    nz = o.tern(p.q, p.theta)[:, c] != 0
    assert nz.any() and (~nz).any()
    assert np.all(np.isnan(r["dX"][:, nz])), "dX rows whose code meets the NaN scale must be NaN"
    if act == "f32":
        assert np.all(np.isnan(r["dX"])), "fp32 path: W_eff = NaN * tern poisons every dX entry"
        assert np.all(np.isnan(o.linear_dx(p.dY, p.q, p.theta, np.where(np.arange(n_out) == c, np.nan,
                                                                          p.scale).astype(np.float32))))
    else:
        assert np.array_equal(r["dX"][:, ~nz], r0["dX"][:, ~nz]), "bf16 fold: a zero code contributes exactly 0"
