"""The SR4 health panel on the GPU (tern_panel_* through the C ABI) against
the oracle's panel: counts bit-exact, scale minimum and maximum exact, the
scale sum to f64 rounding, churn against the previous step's handle."""
import numpy as np
import pytest
import torch

import oracle
import synth
import ternary_weight_linear_tern_amd as tl
from gpu_util import log, to_dev

pytestmark = pytest.mark.gpu

COUNTS = ("total", "neg", "zero", "pos", "rail", "dead", "churn")


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


def _step_q(q, seed):
    """A plausible next q: each entry moves by -1, 0 or +1, clamped to +-7."""
    rng = np.random.default_rng(seed)
    return np.clip(q.astype(np.int16) + rng.integers(-1, 2, size=q.shape), -7, 7).astype(np.int8)


def _check(o, mats, theta, clamp, tag, misaligned=False):
    """mats: list of (q, prev_q or None, scale); the GPU gets prev as a handle."""
    pan = tl.empty_panel()
    tl.tern_panel_reset(pan)
    keep = []
    for q, prev_q, scale in mats:
        n_in, n_out = q.shape
        if misaligned:   # q one byte into a buffer: the byte-wise path
            buf = torch.empty(q.size + 16, dtype=torch.int8, device="cuda")
            qd = buf[1:1 + q.size].view(n_in, n_out)
            qd.copy_(to_dev(q))
        else:
            qd = to_dev(q)
        pk = None
        if prev_q is not None:
            pk = tl.empty_packed(n_in, n_out)
            tl.tern_materialize(to_dev(prev_q), theta, pk)
        sd = to_dev(scale)
        tl.tern_panel_add(qd, theta, sd, pan, prev_packed=pk, q_clamp=clamp)
        keep += [qd, pk, sd]
    torch.cuda.synchronize()
    got = tl.panel_values(pan)
    want = o.panel([(q, None if p is None else o.tern(p, theta), s) for q, p, s in mats], theta, clamp)
    log(f"  {tag}: {[(k, got[k]) for k in COUNTS]}")
    for k in COUNTS:
        assert got[k] == want[k], f"{tag}: {k} {got[k]} != {want[k]}"
    assert got["scale_count"] == want["scale_count"]
    assert got["scale_min"] == want["scale_min"] and got["scale_max"] == want["scale_max"], tag
    assert abs(got["scale_sum"] - want["scale_sum"]) <= 1e-12 * max(1.0, abs(want["scale_sum"])), tag
    for k in ("pct_neg", "pct_zero", "pct_pos", "rail_pct", "dead_pct", "churn_frac"):
        assert got[k] == want[k], f"{tag}: {k}"
    assert abs(got["scale_mean"] - want["scale_mean"]) <= 1e-12 * max(1.0, abs(want["scale_mean"]))
    return pan


@pytest.mark.parametrize("misaligned", [False, True])
def test_panel_matches_oracle(o, misaligned):
    shapes = [(64, 64), (37, 40), (136, 264), (8, 1000), (300, 24), (1, 8)]
    mats = []
    for n, (i, j) in enumerate(shapes):
        q = synth.int8_uniform(synth.stream_seed(9, i, j, n), (i, j), -7, 7)
        q.reshape(-1)[::97] = -128          # out-of-range int8 values are counted as they are
        s = synth.make_inputs(4, i, j, act="f32", config_id=900 + n).scale
        mats.append((_step_q(q, n), q, s))  # post-step q, previous q
    log(f"panel vs oracle, misaligned={misaligned}")
    _check(o, mats, 2, 7, "theta 2", misaligned)
    _check(o, mats, 1, 7, "theta 1", misaligned)
    _check(o, mats, 3, 5, "theta 3 clamp 5", misaligned)
    # the clamp's edges: 0 counts the zeros as rail (never the padding of a
    # ragged row), 128 the int8 value -128
    _check(o, mats, 2, 0, "clamp 0", misaligned)
    _check(o, mats, 2, 128, "clamp 128", misaligned)
    # one matrix without a previous handle: churn is not a fraction of the total
    mixed = [mats[0], (mats[1][0], None, mats[1][2])]
    got = tl.panel_values(_check(o, mixed, 2, 7, "mixed snapshot"))
    assert got["churn_frac"] == 0.0 and got["churn_total"] < got["total"]


def test_panel_large_layer_and_repeatable(o):
    """The six matrices of the Large configuration (50 M weights): exact
    counts, and a second run gives the identical panel."""
    w = synth.WORKLOADS["large"]
    mats = []
    for i, (_, n_in, n_out) in enumerate(w.projs):
        # q and scale of the workload's generator (T = 1: the activations are not needed)
        p = synth.make_inputs(1, n_in, n_out, w.act, w.q_law, w.scale_law, w.theta, w.config_id, i)
        mats.append((_step_q(p.q, 100 + i), p.q, p.scale))
    log("panel: large layer")
    a = _check(o, mats, w.theta, 7, "large")
    b = _check(o, mats, w.theta, 7, "large again")
    assert torch.equal(a, b), "panel differs between identical runs"
