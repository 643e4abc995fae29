"""Hardening of the CPU oracle (test infrastructure, no GPU).

* A sanitizer build: the oracle and the input generator compiled with
  AddressSanitizer and UndefinedBehaviorSanitizer and driven through every
  exported function (tests/csrc/oracle_sanitize.c), including sampled rows and
  columns, zero sizes and the error returns.
* Non-finite inputs: what the plain definitions imply under IEEE arithmetic
  (page "train_gpu.cu": W_eff = scale * tern, then the products; a NaN or an
  Inf times a zero weight is NaN).  A NaN activation poisons exactly its own
  token row of the output and every weight-gradient entry of its feature; a
  NaN scale poisons its own output column and, through W_eff, every input
  gradient; other rows and columns are bitwise those of the clean inputs.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_and_generator_under_sanitizers(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-std=c99", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-ffp-contract=off", "-I", os.path.join(ROOT, "oracle"),
           os.path.join(ROOT, "oracle", "tern_oracle.c"), os.path.join(ROOT, "synth", "synth.c"),
           os.path.join(ROOT, "tests", "csrc", "oracle_sanitize.c"), "-o", exe, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    # the environment is passed on as it is; a library preloaded ahead of the
    # sanitizer runtime is tolerated rather than removed
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "clean under the sanitizers" in r.stdout


@pytest.fixture(scope="module")
def o():
    return oracle.get()


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_nonfinite_activation_poisons_its_row_and_feature(o, act):
    T, n_in, n_out = 9, 16, 24
    p = synth.make_inputs(T, n_in, n_out, act=act, config_id=1401)
    # some zero weights in the poisoned feature's row, so NaN * 0 is exercised
    assert np.any(o.tern(p.q, p.theta)[3] == 0)
    Y0 = o.linear_fwd(p.X, p.q, p.theta, p.scale)
    _, gq0, sg0 = o.linear_wgrad(p.X, p.dY, p.q, p.theta, p.scale)
    X = p.X.copy()
    nan = synth.to_bf16_bits(np.array([np.nan], np.float32))[0] if act == "bf16" else np.float32(np.nan)
    X[5, 3] = nan
    Y = o.linear_fwd(X, p.q, p.theta, p.scale)
    assert np.all(np.isnan(Y[5])), "a NaN activation must poison every output of its token row"
    keep = [t for t in range(T) if t != 5]
    assert np.array_equal(Y[keep], Y0[keep]), "other token rows must not change"
    _, gq, sg = o.linear_wgrad(X, p.dY, p.q, p.theta, p.scale)
    assert np.all(np.isnan(gq[3])), "G[r, :] of the NaN feature r is NaN"
    other = [r for r in range(n_in) if r != 3]
    assert np.array_equal(gq[other], gq0[other])
    assert np.all(np.isnan(sg)), "sgrad sums G[r, c] * tern over all r, including the NaN row"


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_infinite_gradient_poisons_its_row(o, act):
    T, n_in, n_out = 7, 24, 16
    p = synth.make_inputs(T, n_in, n_out, act=act, config_id=1402)
    dX0 = o.linear_dx(p.dY, p.q, p.theta, p.scale)
    dY = p.dY.copy()
    inf = synth.to_bf16_bits(np.array([np.inf], np.float32))[0] if act == "bf16" else np.float32(np.inf)
    dY[2, 6] = inf
    dX = o.linear_dx(dY, p.q, p.theta, p.scale)
    tern_col = o.tern(p.q, p.theta)[:, 6]
    # one infinite term per sum: +-Inf where tern != 0, Inf * 0 = NaN where tern == 0
    assert np.all(np.isinf(dX[2][tern_col != 0])) and np.all(np.isnan(dX[2][tern_col == 0]))
    sign = np.sign(dX[2][tern_col != 0])
    want = np.sign(tern_col[tern_col != 0] * p.scale[6])
    assert np.array_equal(sign, want), "the sign of the infinite input gradient follows W_eff"
    keep = [t for t in range(T) if t != 2]
    assert np.array_equal(dX[keep], dX0[keep])


def test_nan_scale_poisons_its_column_and_every_input_gradient(o):
    T, n_in, n_out = 6, 16, 24
    p = synth.make_inputs(T, n_in, n_out, act="f32", config_id=1403)
    Y0 = o.linear_fwd(p.X, p.q, p.theta, p.scale)
    sc = p.scale.copy()
    sc[4] = np.nan
    Y = o.linear_fwd(p.X, p.q, p.theta, sc)
    assert np.all(np.isnan(Y[:, 4]))
    other = [c for c in range(n_out) if c != 4]
    assert np.array_equal(Y[:, other], Y0[:, other])
    dX = o.linear_dx(p.dY, p.q, p.theta, sc)
    assert np.all(np.isnan(dX)), "W_eff[:, 4] = NaN * tern is NaN even where tern is 0"
    _, gq, sg = o.linear_wgrad(p.X, p.dY, p.q, p.theta, sc)
    assert np.all(np.isnan(gq[:, 4])) and np.all(np.isfinite(gq[:, other]))
    assert np.all(np.isfinite(sg)), "sgrad does not involve the scale"
