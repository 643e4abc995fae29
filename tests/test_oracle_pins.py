"""The oracle against its pins (CPU only)."""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def o():
    return oracle.get()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(o, pin):
    pin(o)


def test_theta_rejected(o):
    with pytest.raises(ValueError):
        o.tern(np.zeros(4, dtype=np.int8), 0)


def test_thread_count_independent(tmp_path):
    """Each output element has a fixed summation order, so results are bitwise
    identical with 1 thread and with many."""
    code = r"""
import sys, numpy as np
sys.path.insert(0, sys.argv[1])
import oracle, synth
o = oracle.get()
p = synth.make_inputs(48, 40, 64, act="bf16", config_id=95)
Y = o.linear_fwd(p.X, p.q, 2, p.scale)
dX = o.linear_dx(p.dY, p.q, 2, p.scale)
G, gq, sg = o.linear_wgrad(p.X, p.dY, p.q, 2, p.scale)
np.savez(sys.argv[2], Y=Y, dX=dX, gq=gq, sg=sg)
"""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    outs = []
    for nt in ("1", "7"):
        f = tmp_path / f"o{nt}.npz"
        env = dict(os.environ, OMP_NUM_THREADS=nt)
        subprocess.run([sys.executable, "-c", code, root, str(f)], check=True, env=env)
        outs.append(np.load(f))
    for k in ("Y", "dX", "gq", "sg"):
        assert np.array_equal(outs[0][k], outs[1][k]), k
