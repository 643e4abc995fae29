"""dX with bf16 activations on shapes with few reduction columns or few
outputs, many seeds, through the C ABI: the scale enters the operand as two
bf16 terms there, so dX meets the 2e-3 gate with a wide margin for every seed
(one rounded term fails it for 10-27 % of the seeds on these shapes)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import ternary_weight_linear_tern_amd as tl
from gpu_util import check_elements, log, rel_l2, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    tl.lib()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("T,n_in,n_out", [(1, 8, 8), (3, 8, 16), (2, 2048, 16), (5, 24, 40), (64, 64, 256),
                                          (1000, 64, 1024), (300, 136, 264)])
def test_dx_small_shapes_many_seeds(T, n_in, n_out):
    o = oracle.get()
    worst = 0.0
    for seed in range(24):
        p = synth.make_inputs(T, n_in, n_out, act="bf16", config_id=8000 + seed,
                              scale_law="lognormal" if seed % 2 else "uniform")
        pk = tl.empty_packed(n_in, n_out)
        tl.tern_materialize(to_dev(p.q), p.theta, pk)
        dX = torch.empty((T, n_in), device="cuda")
        tl.tern_linear_bwd_dx(to_dev(p.dY), pk, to_dev(p.scale), dX)
        got = dX.cpu().numpy()
        want = o.linear_dx(p.dY, p.q, p.theta, p.scale)
        e = rel_l2(got, want)
        worst = max(worst, e)
        assert e <= 2e-5, f"seed {seed}: dX relL2 {e:.3e}"
        check_elements(o, p, {"dX": got}, {"dX": want}, tag=f"dX {T}x{n_in}x{n_out} seed {seed}")
    log(f"  dX {T}x{n_in}x{n_out}: worst relL2 over 24 seeds {worst:.3e}")
