"""CPU oracle for the SR4 ternary projection -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never loads it and shares no code with it.

The arithmetic lives in ``tern_oracle.c`` (plain C99, f64 accumulation, see its
header for the page citations); this module only builds that library with gcc
and marshals numpy arrays through ctypes.

Every function is pinned by the CPU tests in ``tests/test_oracle_*.py``
(hand-derived golden tables, brute force in pure Python, the +-1 sign-matrix
special case against numpy, bilinear identities, finite differences and planted
mutants).  None is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "tern_oracle.c")
LIB = os.path.join(HERE, "liboracle_tern.so")

F32 = 0
BF16 = 1

CFLAGS = ["-std=c99", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off"]


def build(src: str = SRC, out: str = LIB, extra: list[str] | None = None) -> str:
    """Compile the oracle with gcc into a shared library; returns its path."""
    cmd = ["gcc", *CFLAGS, *(extra or []), "-I", HERE, src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


class Oracle:
    """ctypes view of one build of the oracle library."""

    def __init__(self, path: str = LIB):
        if not os.path.exists(path):
            if path != LIB:
                raise FileNotFoundError(path)
            build()
        self.path = path
        L = ctypes.CDLL(path)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        L.oracle_tern.argtypes = [vp, i64, i32, vp]
        L.oracle_tern.restype = ctypes.c_int
        L.oracle_packed_words.argtypes = [i64, i64]
        L.oracle_packed_words.restype = i64
        L.oracle_pack.argtypes = [vp, i64, i64, vp]
        L.oracle_pack.restype = ctypes.c_int
        L.oracle_unpack.argtypes = [vp, i64, i64, vp]
        L.oracle_unpack.restype = ctypes.c_int
        L.oracle_widen.argtypes = [vp, i32, i64, vp]
        L.oracle_widen.restype = None
        L.oracle_linear_fwd.argtypes = [vp, i32, vp, i32, vp, i64, i64, i64, vp, i64, vp]
        L.oracle_linear_fwd.restype = ctypes.c_int
        L.oracle_linear_dx.argtypes = [vp, i32, vp, i32, vp, i64, i64, i64, vp, i64, vp]
        L.oracle_linear_dx.restype = ctypes.c_int
        L.oracle_linear_wgrad.argtypes = [vp, vp, i32, vp, i32, vp, i64, i64, i64, vp, i64,
                                          vp, vp, vp]
        L.oracle_linear_wgrad.restype = ctypes.c_int
        L.oracle_panel_add.argtypes = [vp, i64, i64, i32, i32, vp, vp, vp, vp]
        L.oracle_panel_add.restype = ctypes.c_int
        f64 = ctypes.c_double
        L.oracle_scale_adamw.argtypes = [vp, vp, vp, vp, i64, i32, f64, f64, f64, f64, f64, f64]
        L.oracle_scale_adamw.restype = ctypes.c_int
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_set_num_threads.argtypes = [ctypes.c_int]
        L.oracle_set_num_threads.restype = ctypes.c_int
        self.L = L

    # -- helpers --------------------------------------------------------
    @staticmethod
    def _p(a):
        return None if a is None else a.ctypes.data_as(ctypes.c_void_p)

    @staticmethod
    def _act(a):
        """Return (contiguous array, dtype code) for an fp32 or bf16-bit array."""
        a = np.ascontiguousarray(a)
        if a.dtype == np.float32:
            return a, F32
        if a.dtype == np.uint16:
            return a, BF16
        raise TypeError(f"activation must be float32 or uint16 (bf16 bits), got {a.dtype}")

    def num_threads(self) -> int:
        return int(self.L.oracle_num_threads())

    def set_num_threads(self, n: int) -> int:
        """Use n threads from now on; returns the count in effect."""
        return int(self.L.oracle_set_num_threads(int(n)))

    # -- ternarisation and packing -----------------------------------------
    def tern(self, q: np.ndarray, theta: int) -> np.ndarray:
        q = np.ascontiguousarray(q, dtype=np.int8)
        out = np.empty(q.shape, dtype=np.int8)
        rc = self.L.oracle_tern(self._p(q), q.size, int(theta), self._p(out))
        if rc != 0:
            raise ValueError(f"oracle_tern: theta {theta} rejected")
        return out

    def packed_words(self, n_in: int, n_out: int) -> int:
        return int(self.L.oracle_packed_words(n_in, n_out))

    def pack(self, tern: np.ndarray) -> np.ndarray:
        tern = np.ascontiguousarray(tern, dtype=np.int8)
        n_in, n_out = tern.shape
        wpr = (n_out + 15) // 16
        out = np.empty((n_in, wpr), dtype=np.uint32)
        if self.L.oracle_pack(self._p(tern), n_in, n_out, self._p(out)) != 0:
            raise ValueError("oracle_pack: value outside {-1,0,1}")
        return out

    def unpack(self, packed: np.ndarray, n_in: int, n_out: int) -> np.ndarray:
        packed = np.ascontiguousarray(packed, dtype=np.uint32)
        out = np.empty((n_in, n_out), dtype=np.int8)
        if self.L.oracle_unpack(self._p(packed), n_in, n_out, self._p(out)) != 0:
            raise ValueError("oracle_unpack: reserved or nonzero padding code")
        return out

    def panel(self, mats, theta: int, q_clamp: int = 7) -> dict:
        """SR4 health panel over the matrices `mats`, a list of (q, prev_tern or
        None, scale).  Returns the counts and the page's fractions: churn only
        when every matrix has a previous classification."""
        counts = np.zeros(7, dtype=np.int64)
        sstat = np.array([0.0, 0.0, np.inf, -np.inf])
        snap_valid = True
        for q, prev, scale in mats:
            q = np.ascontiguousarray(q, dtype=np.int8)
            n_in, n_out = q.shape
            prev = None if prev is None else np.ascontiguousarray(prev, dtype=np.int8)
            snap_valid = snap_valid and prev is not None
            scale = np.ascontiguousarray(scale, dtype=np.float32)
            if self.L.oracle_panel_add(self._p(q), n_in, n_out, int(theta), int(q_clamp), self._p(prev),
                                       self._p(scale), self._p(counts), self._p(sstat)) != 0:
                raise ValueError(f"oracle_panel_add: theta {theta} rejected")
        names = ("total", "neg", "zero", "pos", "rail", "dead", "churn")
        r = {k: int(v) for k, v in zip(names, counts)}
        dt = float(r["total"]) if r["total"] else 1.0
        r.update(pct_neg=r["neg"] / dt, pct_zero=r["zero"] / dt, pct_pos=r["pos"] / dt,
                 rail_pct=r["rail"] / dt, dead_pct=r["dead"] / dt,
                 churn_frac=(r["churn"] / dt) if snap_valid else 0.0,
                 scale_count=int(sstat[0]), scale_sum=float(sstat[1]),
                 scale_mean=float(sstat[1] / sstat[0]) if sstat[0] else 0.0,
                 scale_min=float(sstat[2]) if sstat[0] else 0.0,
                 scale_max=float(sstat[3]) if sstat[0] else 0.0)
        return r

    def scale_adamw(self, sgrad, scale, m, v, t, lr, scale_lr, b1=0.9, b2=0.999, eps=1e-8, wd=0.0):
        """One AdamW step of the per-column scale; returns new (scale, m, v)
        as float64 arrays (the inputs are not modified)."""
        g = np.ascontiguousarray(sgrad, dtype=np.float64)
        sc = np.array(scale, dtype=np.float64)
        mm = np.array(m, dtype=np.float64)
        vv = np.array(v, dtype=np.float64)
        if self.L.oracle_scale_adamw(self._p(g), self._p(sc), self._p(mm), self._p(vv), g.size, int(t),
                                     float(lr), float(scale_lr), float(b1), float(b2), float(eps),
                                     float(wd)) != 0:
            raise ValueError(f"oracle_scale_adamw: step {t} rejected")
        return sc, mm, vv

    def widen(self, a: np.ndarray) -> np.ndarray:
        a, dt = self._act(a)
        out = np.empty(a.shape, dtype=np.float64)
        self.L.oracle_widen(self._p(a), dt, a.size, self._p(out))
        return out

    # -- the projection ---------------------------------------------------
    def linear_fwd(self, X, q, theta, scale, rows=None) -> np.ndarray:
        X, dt = self._act(X)
        T, n_in = X.shape
        q = np.ascontiguousarray(q, dtype=np.int8)
        n_out = q.shape[1]
        assert q.shape[0] == n_in
        scale = np.ascontiguousarray(scale, dtype=np.float32)
        rws = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
        nr = T if rws is None else rws.size
        Y = np.empty((nr, n_out), dtype=np.float64)
        rc = self.L.oracle_linear_fwd(self._p(X), dt, self._p(q), int(theta), self._p(scale),
                                      T, n_in, n_out, self._p(rws), nr, self._p(Y))
        if rc != 0:
            raise ValueError(f"oracle_linear_fwd rc={rc}")
        return Y

    def linear_dx(self, dY, q, theta, scale, rows=None) -> np.ndarray:
        dY, dt = self._act(dY)
        T, n_out = dY.shape
        q = np.ascontiguousarray(q, dtype=np.int8)
        n_in = q.shape[0]
        assert q.shape[1] == n_out
        scale = np.ascontiguousarray(scale, dtype=np.float32)
        rws = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
        nr = T if rws is None else rws.size
        dX = np.empty((nr, n_in), dtype=np.float64)
        rc = self.L.oracle_linear_dx(self._p(dY), dt, self._p(q), int(theta), self._p(scale),
                                     T, n_in, n_out, self._p(rws), nr, self._p(dX))
        if rc != 0:
            raise ValueError(f"oracle_linear_dx rc={rc}")
        return dX

    def linear_wgrad(self, X, dY, q, theta, scale, cols=None, want_G=False):
        """Returns (G or None, gq, sgrad) for the selected output columns."""
        X, dt = self._act(X)
        dY, dt2 = self._act(dY)
        assert dt == dt2, "X and dY must share a storage type"
        T, n_in = X.shape
        n_out = dY.shape[1]
        assert dY.shape[0] == T
        q = np.ascontiguousarray(q, dtype=np.int8)
        assert q.shape == (n_in, n_out)
        scale = np.ascontiguousarray(scale, dtype=np.float32)
        cls = None if cols is None else np.ascontiguousarray(cols, dtype=np.int64)
        nc = n_out if cls is None else cls.size
        G = np.empty((n_in, nc), dtype=np.float64) if want_G else None
        gq = np.empty((n_in, nc), dtype=np.float64)
        sg = np.empty((nc,), dtype=np.float64)
        rc = self.L.oracle_linear_wgrad(self._p(X), self._p(dY), dt, self._p(q), int(theta),
                                        self._p(scale), T, n_in, n_out, self._p(cls), nc,
                                        self._p(G), self._p(gq), self._p(sg))
        if rc != 0:
            raise ValueError(f"oracle_linear_wgrad rc={rc}")
        return G, gq, sg


_default: Oracle | None = None


def get() -> Oracle:
    """The default build of the oracle (compiled on first use if missing)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
