"""Host-side argument checks, on the CPU (no GPU, nothing launched).

* The planner's launch check (tern_plan.cpp, built with g++ and the
  sanitizers): a missing operand, output, fragment copy or -- where the dW
  epilogue writes it -- sgrad partial table is refused before any kernel is
  enqueued; a workspace limit lowers the dW split count until the plan fits.
* The Python binding: tensors whose dtype, shape or size do not match the
  call are refused with TypeError / ValueError before the C library sees a
  pointer, and so are host (CPU) tensors.
"""
import os
import shutil
import subprocess

import pytest
import torch

import ternary_weight_linear_tern_amd as tl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_planner_launch_checks(tmp_path):
    if not shutil.which("g++"):
        pytest.skip("g++ not available")
    exe = str(tmp_path / "plan_check")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "tests", "csrc", "plan_check.cpp"),
           os.path.join(ROOT, "ternary_weight_linear_tern_amd", "csrc", "tern_plan.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="verify_asan_link_order=0")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(tl.LIB_PATH):
        from ternary_weight_linear_tern_amd import build
        build.build()
    return tl.lib()


def _t(shape, dtype=torch.float32):
    return torch.zeros(shape, dtype=dtype)


def _proj(T=16, n_in=32, n_out=48, act=torch.bfloat16):
    return dict(X=_t((T, n_in), act), dY=_t((T, n_out), act), q=_t((n_in, n_out), torch.int8),
                scale=_t((n_out,)), packed=_t((tl.tern_packed_words(n_in, n_out),), torch.int32),
                Y=_t((T, n_out)), dX=_t((T, n_in)), gq=_t((n_in, n_out)), sgrad=_t((n_out,)),
                ws=_t((tl.tern_linear_bwd_workspace_bytes(T, n_in, n_out) + 16,), torch.uint8))


def _refused(fn, *args, **kw):
    """Refused for the mismatch itself: the device test comes last, so a
    refusal that names the GPU means the mismatch went unnoticed."""
    with pytest.raises((TypeError, ValueError)) as e:
        fn(*args, **kw)
    assert "GPU" not in str(e.value), f"mismatch not detected: {e.value}"


def test_binding_rejects_mismatched_tensors(L):
    d = _proj()
    X, dY, pk, sc, Y, dX, gq, sg, ws = (d[k] for k in ("X", "dY", "packed", "scale", "Y", "dX", "gq", "sgrad",
                                                        "ws"))
    # forward: Y of the wrong width, fp32 Y with a wrong dtype, bf16 Y from fp32 X, short handle
    _refused(tl.tern_linear_fwd, X, pk, sc, _t((16, 40)))
    _refused(tl.tern_linear_fwd, X, pk, sc, _t((16, 48), torch.float16))
    _refused(tl.tern_linear_fwd, X.float(), pk, sc, _t((16, 48), torch.bfloat16))
    _refused(tl.tern_linear_fwd, X, pk[:-1], sc, Y)
    _refused(tl.tern_linear_fwd, X, pk.view(torch.uint8), sc, Y)
    _refused(tl.tern_linear_fwd, X, pk, sc.double(), Y)
    # backward: fp32 X with bf16 dY (the kernels would read T*out*4 bytes of a
    # T*out*2 buffer), wrong dX / gq / sgrad shapes, a bf16 dX
    _refused(tl.tern_linear_bwd, X.float(), dY, pk, sc, dX, gq, sg, ws)
    _refused(tl.tern_linear_bwd, X, dY[:, :40], pk, sc, dX, gq, sg, ws)
    _refused(tl.tern_linear_bwd, X, dY, pk, sc, dX[:8], gq, sg, ws)
    _refused(tl.tern_linear_bwd, X, dY, pk, sc, dX, gq[:, :40], sg, ws)
    _refused(tl.tern_linear_bwd, X, dY, pk, sc, dX, gq, sg[:40], ws)
    _refused(tl.tern_linear_bwd, X, dY, pk, sc, dX.bfloat16(), gq, sg, ws)
    _refused(tl.tern_linear_bwd_dx, dY, pk, sc, _t((16, 32), torch.bfloat16))
    _refused(tl.tern_linear_bwd_dx, dY, pk, sc[:40], dX)
    _refused(tl.tern_linear_bwd_dw, X, dY.float(), pk, sc, gq, sg, ws)
    _refused(tl.tern_linear_bwd_dw, X, dY, pk[:10], sc, gq, sg, ws)
    _refused(tl.tern_linear_bwd_dx_acc, dY, pk, sc, dX.double())
    _refused(tl.tern_linear_bwd_dw_acc, X, dY, pk, sc, gq.double(), sg, ws, 0.5)
    # materialize: q not int8, short handle
    _refused(tl.tern_materialize, d["q"].to(torch.int16), 2, pk)
    _refused(tl.tern_materialize, d["q"], 2, pk[:100])
    # group gather: a member with the wrong row count, a short group buffer
    q2 = _t((32, 16), torch.int8)
    _refused(tl.tern_group_gather, [d["q"], _t((24, 16), torch.int8)], [sc, _t((16,))], _t((32, 64), torch.int8),
             _t((64,)))
    _refused(tl.tern_group_gather, [d["q"], q2], [sc, _t((16,))], _t((32, 60), torch.int8), _t((64,)))
    # scale step and panel
    _refused(tl.tern_scale_adamw, sg, sc, _t((40,)), _t((48,)), 1, 1e-3)
    _refused(tl.tern_panel_add, d["q"], 2, sc, _t((12,), torch.float32))
    _refused(tl.tern_panel_add, d["q"], 2, sc[:40], _t((12,), torch.float64))


def test_binding_rejects_host_tensors(L):
    """Consistent shapes and dtypes, but host memory: refused before any
    pointer reaches the library (a host address would fault the GPU)."""
    d = _proj()
    with pytest.raises(ValueError, match="GPU"):
        tl.tern_linear_fwd(d["X"], d["packed"], d["scale"], d["Y"])
    with pytest.raises(ValueError, match="GPU"):
        tl.tern_linear_bwd(d["X"], d["dY"], d["packed"], d["scale"], d["dX"], d["gq"], d["sgrad"], d["ws"])
    with pytest.raises(ValueError, match="GPU"):
        tl.tern_materialize(d["q"], 2, d["packed"])


def test_panel_fractions_on_the_host(L):
    """The page's fractions come from the library's host function."""
    counts = dict(total=200, neg=50, zero=70, pos=80, rail=20, dead=70, churn=30, churn_total=200,
                  scale_count=8)
    h = torch.zeros(12, dtype=torch.float64)
    h[:9].view(torch.int64)[:] = torch.tensor([counts[k] for k in tl.PANEL_COUNTS])
    h[9:] = torch.tensor([0.4, 0.01, 0.1], dtype=torch.float64)
    f = tl.tern_panel_fractions(h)
    assert f == dict(pct_neg=0.25, pct_zero=0.35, pct_pos=0.4, rail_pct=0.1, dead_pct=0.35, churn_frac=0.15,
                     scale_mean=0.05)
    h[:9].view(torch.int64)[7] = 150   # some elements had no previous handle: no churn fraction
    assert tl.tern_panel_fractions(h)["churn_frac"] == 0.0
    assert all(v == 0.0 for v in tl.tern_panel_fractions(torch.zeros(12, dtype=torch.float64)).values())
    assert L.tern_panel_fractions(None, None) == -1
