"""Seeded synthetic inputs for the ternary projection (no method arithmetic).

The element generators live in ``synth.c`` (SplitMix64 counter streams,
Box-Muller normals, Lemire integer ranges, RNE bf16).  This module builds that
library, defines the benchmark workloads and hands out numpy arrays:

* activations as ``float32`` (fp32 workloads) or ``uint16`` holding bf16 bits;
* ``q`` as ``int8 [in, out]`` (row-major, rows = input dim, cols = output dim);
* ``scale`` as ``float32 [out]``.

Both the HIP path and the oracle receive exactly these arrays; neither side
generates its own inputs.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "synth.c")
LIB = os.path.join(HERE, "libsynth.so")

SEED_ACT = 1234  # activations and scale
SEED_Q = 42      # ternary accumulators
TENSOR_X, TENSOR_DY, TENSOR_Q, TENSOR_SCALE = 0, 1, 2, 3


def build(out: str = LIB) -> str:
    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-fopenmp", SRC, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


_lib = None


def _L():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        u64, i64, i32, vp, d = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32,
                                ctypes.c_void_p, ctypes.c_double)
        L.synth_stream_seed.argtypes = [u64, u64, u64, u64]
        L.synth_stream_seed.restype = u64
        L.synth_u64.argtypes = [u64, u64]
        L.synth_u64.restype = u64
        for name in ("synth_normal_f32", "synth_normal_bf16", "synth_uniform_f32",
                     "synth_lognormal_f32"):
            getattr(L, name).argtypes = [u64, i64, d, d, vp]
            getattr(L, name).restype = None
        L.synth_int8_uniform.argtypes = [u64, i64, i32, i32, vp]
        L.synth_int8_zero_or_pm.argtypes = [u64, i64, d, i32, i32, vp]
        L.synth_f32_to_bf16.argtypes = [vp, i64, vp]
        L.synth_sample_indices.argtypes = [u64, i64, i64, vp]
        _lib = L
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def stream_seed(base: int, config_id: int, proj_id: int, tensor_id: int) -> int:
    return int(_L().synth_stream_seed(base, config_id, proj_id, tensor_id))


def normal(seed: int, shape, mean=0.0, std=1.0, bf16=False) -> np.ndarray:
    n = int(np.prod(shape))
    if bf16:
        a = np.empty(shape, dtype=np.uint16)
        _L().synth_normal_bf16(seed, n, mean, std, _ptr(a))
    else:
        a = np.empty(shape, dtype=np.float32)
        _L().synth_normal_f32(seed, n, mean, std, _ptr(a))
    return a


def uniform(seed: int, shape, lo: float, hi: float) -> np.ndarray:
    a = np.empty(shape, dtype=np.float32)
    _L().synth_uniform_f32(seed, int(np.prod(shape)), lo, hi, _ptr(a))
    return a


def lognormal(seed: int, shape, mu: float, sigma: float) -> np.ndarray:
    a = np.empty(shape, dtype=np.float32)
    _L().synth_lognormal_f32(seed, int(np.prod(shape)), mu, sigma, _ptr(a))
    return a


def int8_uniform(seed: int, shape, lo: int, hi: int) -> np.ndarray:
    a = np.empty(shape, dtype=np.int8)
    _L().synth_int8_uniform(seed, int(np.prod(shape)), lo, hi, _ptr(a))
    return a


def int8_zero_or_pm(seed: int, shape, p_zero: float, mag_lo: int, mag_hi: int) -> np.ndarray:
    a = np.empty(shape, dtype=np.int8)
    _L().synth_int8_zero_or_pm(seed, int(np.prod(shape)), p_zero, mag_lo, mag_hi, _ptr(a))
    return a


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    _L().synth_f32_to_bf16(_ptr(a), a.size, _ptr(out))
    return out


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits, for building test inputs."""
    return (np.ascontiguousarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def sample_indices(seed: int, n: int, rng: int) -> np.ndarray:
    a = np.empty((n,), dtype=np.int64)
    _L().synth_sample_indices(seed, n, rng, _ptr(a))
    return np.unique(a)


# --------------------------------------------------------------------------
# Workloads: one layer's ternary projections of an RWKV-x style block.  Rows of
# q are the input dim, columns the output dim; every projection has its own
# activations (time-mix projections read different token-shift mixes).
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    name: str
    config_id: int
    T: int
    projs: tuple  # ((name, in, out), ...)
    act: str      # "f32" or "bf16"
    q_law: str    # "uniform" (U{-7..7}) or "skewed" (30% zeros, else +-U{1..7})
    scale_law: str  # "uniform" (U[0.01, 0.1]) or "lognormal" (ln 0.02, 0.5)
    theta: int = 2
    note: str = ""

    @property
    def sum_in_out(self) -> int:
        return sum(i * o for _, i, o in self.projs)

    @property
    def flops(self) -> int:
        """Algorithmic flops of one fwd + bwd over all projections."""
        return 6 * self.T * self.sum_in_out


def _block(d: int, ffn: int):
    return (("receptance", d, d), ("key", d, d), ("value", d, d), ("output", d, d),
            ("ffn_key", d, ffn), ("ffn_value", ffn, d))


WORKLOADS = {
    "tiny": Workload("tiny", 0, 64, (("proj", 64, 64),), "f32", "uniform", "uniform",
                     note="T=64, 64->64, fp32"),
    "rwkv_small": Workload("rwkv_small", 1, 2048, _block(512, 2048), "bf16", "uniform",
                           "uniform", note="batch 8 x ctx 256, d=512, ffn 2048"),
    "mid": Workload("mid", 2, 8192, _block(1024, 4096), "bf16", "skewed", "uniform",
                    note="T=8192, d=1024, ffn 4096, skewed q"),
    "large": Workload("large", 3, 16384, _block(2048, 8192), "bf16", "uniform", "uniform",
                      note="T=16384 (16 x 1024), d=2048, ffn 8192"),
    "largest": Workload("largest", 4, 32768, _block(4096, 16384), "bf16", "uniform",
                        "lognormal", note="T=32768, d=4096, ffn 16384, lognormal scale"),
}


@dataclass
class ProjInputs:
    X: np.ndarray
    dY: np.ndarray
    q: np.ndarray
    scale: np.ndarray
    theta: int
    act: str
    name: str = ""
    meta: dict = field(default_factory=dict)


def make_inputs(T: int, n_in: int, n_out: int, act: str = "bf16", q_law: str = "uniform",
                scale_law: str = "uniform", theta: int = 2, config_id: int = 99,
                proj_id: int = 0, name: str = "") -> ProjInputs:
    bf = act == "bf16"
    X = normal(stream_seed(SEED_ACT, config_id, proj_id, TENSOR_X), (T, n_in), 0.0, 1.0, bf)
    dY = normal(stream_seed(SEED_ACT, config_id, proj_id, TENSOR_DY), (T, n_out), 0.0, 0.01, bf)
    qs = stream_seed(SEED_Q, config_id, proj_id, TENSOR_Q)
    if q_law == "uniform":
        q = int8_uniform(qs, (n_in, n_out), -7, 7)
    elif q_law == "skewed":
        q = int8_zero_or_pm(qs, (n_in, n_out), 0.3, 1, 7)
    else:
        raise ValueError(q_law)
    ss = stream_seed(SEED_ACT, config_id, proj_id, TENSOR_SCALE)
    if scale_law == "uniform":
        scale = uniform(ss, (n_out,), 0.01, 0.1)
    elif scale_law == "lognormal":
        scale = lognormal(ss, (n_out,), math.log(0.02), 0.5)
    else:
        raise ValueError(scale_law)
    return ProjInputs(X, dY, q, scale, theta, act, name,
                      dict(T=T, n_in=n_in, n_out=n_out, q_law=q_law, scale_law=scale_law))


def workload_inputs(w: Workload, proj_index: int) -> ProjInputs:
    name, n_in, n_out = w.projs[proj_index]
    return make_inputs(w.T, n_in, n_out, w.act, w.q_law, w.scale_law, w.theta,
                       w.config_id, proj_index, name)
