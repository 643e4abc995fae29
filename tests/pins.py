"""Pins of the CPU oracle against facts that do not come from the oracle.

Each ``pin_*`` takes an ``oracle.Oracle`` (the default build, or a build with a
planted mistake) and raises ``AssertionError`` when the oracle disagrees with:

* hand-derived golden tables (tests/golden/, each citing the page's rule);
* brute force written independently in pure Python on tiny shapes;
* the +-1 sign-matrix special case (scale = 1, every |q| >= theta), which is a
  plain matrix product computed by numpy;
* identities of the bilinear form L = <dY, X . W_eff> that hold exactly in real
  arithmetic (five ways of writing L, and sgrad[c] = <dY[:,c], Y[:,c]> / scale[c]);
* finite differences of L, which is exactly linear in scale, X and tern, so a
  central difference (or a single tern flip) equals the gradient up to rounding;
* the degenerate case theta > max|q| (tern all zero).

The inputs here are crafted with numpy / the synth generator; nothing comes from
the HIP library.
"""
from __future__ import annotations

import os

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden_kv(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, *v = line.split()
            out.setdefault(k, []).append(v)
    return out


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    if nb == 0:
        return 0.0 if np.all(a == 0) else np.inf
    return float(np.linalg.norm(a - b) / nb)


# ---------------------------------------------------------------------------
# ternarisation and packing
# ---------------------------------------------------------------------------

def pin_tern_golden(o):
    qs = list(range(-8, 9)) + [-128, 127]
    with open(os.path.join(GOLDEN, "tern_rule.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            vals = [int(v) for v in line.split()]
            theta, want = vals[0], vals[1:]
            got = o.tern(np.array(qs, dtype=np.int8), theta)
            assert list(got) == want, f"theta={theta}: {list(got)} != {want}"


def pin_tern_properties(o):
    q = np.arange(-128, 128, dtype=np.int8)
    for theta in range(1, 9):
        t = o.tern(q, theta).astype(np.int64)
        qi = q.astype(np.int64)
        assert set(np.unique(t)) <= {-1, 0, 1}
        assert np.all(np.diff(t) >= 0), "tern must be non-decreasing in q"
        assert np.all((t == 0) == (np.abs(qi) < theta)), "dead zone is |q| < theta"
        nz = t != 0
        assert np.all(np.sign(qi[nz]) == t[nz]), "outside the dead zone tern = sign(q)"
        # odd symmetry on -127..127
        m = qi > -128
        assert np.all(o.tern(-q[m], theta).astype(np.int64) == -t[m])


def pin_pack_golden(o):
    g = _golden_kv("pack_words.txt")
    n_in, n_out = int(g["in"][0][0]), int(g["out"][0][0])
    tern = np.array([[int(v) for v in row] for row in g["tern"]], dtype=np.int8)
    want = np.array([int(v, 16) for v in g["words"][0]], dtype=np.uint32).reshape(n_in, -1)
    got = o.pack(tern)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.array_equal(got, want), [hex(int(x)) for x in got.ravel()]
    assert np.array_equal(o.unpack(want, n_in, n_out), tern)
    assert o.packed_words(n_in, n_out) == want.size


def pin_pack_roundtrip(o):
    for (n_in, n_out) in [(1, 1), (3, 15), (5, 16), (7, 17), (4, 33), (9, 64), (2, 100)]:
        q = synth.int8_uniform(synth.stream_seed(7, n_in, n_out, 0), (n_in, n_out), -7, 7)
        t = o.tern(q, 2)
        p = o.pack(t)
        assert p.shape == (n_in, (n_out + 15) // 16)
        assert np.array_equal(o.unpack(p, n_in, n_out), t)
        # independent decode of the format: 2-bit field (r, c) at bits 2*(c%16) of word c/16
        for r in range(n_in):
            for c in range(n_out):
                code = (int(p[r, c // 16]) >> (2 * (c % 16))) & 3
                assert code == {0: 0, 1: 1, -1: 3}[int(t[r, c])]
            for c in range(n_out, p.shape[1] * 16):
                assert (int(p[r, c // 16]) >> (2 * (c % 16))) & 3 == 0, "padding must be 00"


# ---------------------------------------------------------------------------
# the projection
# ---------------------------------------------------------------------------

def pin_worked_example(o):
    g = _golden_kv("worked_example.txt")
    T, n_in, n_out = int(g["T"][0][0]), int(g["in"][0][0]), int(g["out"][0][0])
    theta = int(g["theta"][0][0])
    f = lambda k, shape: np.array([float(v) for v in g[k][0]]).reshape(shape)
    q = f("q", (n_in, n_out)).astype(np.int8)
    scale = f("scale", (n_out,)).astype(np.float32)
    X = f("X", (T, n_in)).astype(np.float32)
    dY = f("dY", (T, n_out)).astype(np.float32)
    Y = o.linear_fwd(X, q, theta, scale)
    dX = o.linear_dx(dY, q, theta, scale)
    G, gq, sg = o.linear_wgrad(X, dY, q, theta, scale, want_G=True)
    assert np.array_equal(Y, f("Y", (T, n_out))), Y
    assert np.array_equal(dX, f("dX", (T, n_in))), dX
    assert np.array_equal(G, f("G", (n_in, n_out))), G
    assert np.array_equal(gq, f("gq", (n_in, n_out))), gq
    assert np.array_equal(sg, f("sgrad", (n_out,))), sg
    # the same example through bf16 storage (all values are exact in bf16)
    Yb = o.linear_fwd(synth.to_bf16_bits(X), q, theta, scale)
    assert np.array_equal(Yb, Y)


def _brute(X, dY, q, theta, scale):
    """Independent pure-Python loops over the definitions."""
    T, n_in = len(X), len(X[0])
    n_out = len(scale)
    tern = [[(1 if q[r][c] >= theta else (-1 if q[r][c] <= -theta else 0))
             for c in range(n_out)] for r in range(n_in)]
    W = [[float(scale[c]) * tern[r][c] for c in range(n_out)] for r in range(n_in)]
    Y = [[sum(X[t][r] * W[r][c] for r in range(n_in)) for c in range(n_out)] for t in range(T)]
    dX = [[sum(dY[t][c] * W[r][c] for c in range(n_out)) for r in range(n_in)] for t in range(T)]
    G = [[sum(X[t][r] * dY[t][c] for t in range(T)) for c in range(n_out)] for r in range(n_in)]
    gq = [[G[r][c] * float(scale[c]) for c in range(n_out)] for r in range(n_in)]
    sg = [sum(G[r][c] * tern[r][c] for r in range(n_in)) for c in range(n_out)]
    return Y, dX, G, gq, sg


def pin_brute_force(o):
    shapes = [(1, 1, 1), (2, 3, 16), (3, 5, 32), (5, 7, 9), (4, 16, 3), (6, 12, 20)]
    for i, (T, n_in, n_out) in enumerate(shapes):
        for act in ("f32", "bf16"):
            p = synth.make_inputs(T, n_in, n_out, act=act, config_id=50 + i)
            Xf = p.X if act == "f32" else synth.bf16_bits_to_f32(p.X)
            dYf = p.dY if act == "f32" else synth.bf16_bits_to_f32(p.dY)
            Xl = [[float(v) for v in row] for row in Xf]
            dYl = [[float(v) for v in row] for row in dYf]
            ql = [[int(v) for v in row] for row in p.q]
            Y, dX, G, gq, sg = _brute(Xl, dYl, ql, p.theta, p.scale)
            assert _rel(o.linear_fwd(p.X, p.q, p.theta, p.scale), Y) < 1e-13
            assert _rel(o.linear_dx(p.dY, p.q, p.theta, p.scale), dX) < 1e-13
            oG, ogq, osg = o.linear_wgrad(p.X, p.dY, p.q, p.theta, p.scale, want_G=True)
            assert _rel(oG, G) < 1e-13
            assert _rel(ogq, gq) < 1e-13
            assert _rel(osg, sg) < 1e-12


def pin_sign_matrix_gemm(o):
    """scale = 1 and |q| >= theta everywhere: W_eff is a +-1 matrix S and every
    output is a plain product (numpy matmul)."""
    for i, (T, n_in, n_out) in enumerate([(8, 16, 16), (33, 40, 24), (64, 64, 64)]):
        p = synth.make_inputs(T, n_in, n_out, act="f32", config_id=60 + i)
        mag = synth.int8_uniform(synth.stream_seed(3, i, 0, 0), (n_in, n_out), 2, 7)
        sgn = synth.int8_uniform(synth.stream_seed(3, i, 0, 1), (n_in, n_out), 0, 1)
        q = np.where(sgn == 1, mag, -mag).astype(np.int8)
        S = np.where(sgn == 1, 1.0, -1.0)
        one = np.ones(n_out, dtype=np.float32)
        X = p.X.astype(np.float64)
        dY = p.dY.astype(np.float64)
        assert _rel(o.linear_fwd(p.X, q, 2, one), X @ S) < 1e-13
        assert _rel(o.linear_dx(p.dY, q, 2, one), dY @ S.T) < 1e-13
        G, gq, sg = o.linear_wgrad(p.X, p.dY, q, 2, one, want_G=True)
        Gn = X.T @ dY
        assert _rel(G, Gn) < 1e-13
        assert _rel(gq, Gn) < 1e-13
        assert _rel(sg, (Gn * S).sum(axis=0)) < 1e-12


def pin_bilinear_identities(o):
    """<dY, Y> = <X, dX> = <G, W_eff> = sum_c scale[c] sgrad[c] = <gq, tern>, and
    sgrad[c] = <dY[:,c], Y[:,c]> / scale[c]."""
    for i, (T, n_in, n_out, act, ql) in enumerate([(17, 24, 40, "f32", "uniform"),
                                                  (50, 33, 16, "bf16", "skewed"),
                                                  (64, 64, 64, "bf16", "uniform")]):
        p = synth.make_inputs(T, n_in, n_out, act=act, q_law=ql, config_id=70 + i)
        X = o.widen(p.X)
        dY = o.widen(p.dY)
        tern = o.tern(p.q, p.theta).astype(np.float64)
        Y = o.linear_fwd(p.X, p.q, p.theta, p.scale)
        dX = o.linear_dx(p.dY, p.q, p.theta, p.scale)
        G, gq, sg = o.linear_wgrad(p.X, p.dY, p.q, p.theta, p.scale, want_G=True)
        W = tern * p.scale.astype(np.float64)[None, :]
        forms = [np.sum(dY * Y), np.sum(X * dX), np.sum(G * W),
                 np.sum(p.scale.astype(np.float64) * sg), np.sum(gq * tern)]
        ref = forms[0]
        for k, v in enumerate(forms[1:], 1):
            assert abs(v - ref) <= 1e-11 * max(1.0, abs(ref)) + 1e-12, (k, v, ref)
        col = np.sum(dY * Y, axis=0) / p.scale.astype(np.float64)
        assert _rel(sg, col) < 1e-10


def pin_finite_differences(o):
    """L(s) = <dY, X . W_eff(s)> is linear in scale, in X and in tern, so central
    differences (steps of 2% and 8%, as a parity check of a gradient) and single
    tern flips reproduce sgrad, dX and gq up to rounding."""
    T, n_in, n_out = 24, 20, 32
    p = synth.make_inputs(T, n_in, n_out, act="f32", config_id=80)

    def L(X, q, scale):
        Y = o.linear_fwd(X, q, p.theta, scale)
        return float(np.sum(p.dY.astype(np.float64) * Y))

    dX = o.linear_dx(p.dY, p.q, p.theta, p.scale)
    G, gq, sg = o.linear_wgrad(p.X, p.dY, p.q, p.theta, p.scale, want_G=True)
    big = list(np.argsort(-np.abs(sg))[:4]) + [3, 11, 17, 29]
    for c in big:
        for frac in (0.02, 0.08):
            s0 = float(p.scale[c])
            h = frac * s0
            sp = p.scale.astype(np.float64).copy()
            sm = sp.copy()
            sp[c] = s0 + h
            sm[c] = s0 - h
            # scale is stored in fp32: use the exact fp32 step actually taken
            spf, smf = sp.astype(np.float32), sm.astype(np.float32)
            hh = (float(spf[c]) - float(smf[c])) / 2
            fd = (L(p.X, p.q, spf) - L(p.X, p.q, smf)) / (2 * hh)
            assert abs(fd - sg[c]) <= 1e-9 * max(1e-3, abs(sg[c])) + 1e-12, (c, fd, sg[c])
    # input gradient, a few coordinates
    for (t, r) in [(0, 0), (5, 7), (23, 19), (11, 3)]:
        h = 0.05
        Xp = p.X.copy()
        Xm = p.X.copy()
        Xp[t, r] += np.float32(h)
        Xm[t, r] -= np.float32(h)
        hh = (float(Xp[t, r]) - float(Xm[t, r])) / 2
        fd = (L(Xp, p.q, p.scale) - L(Xm, p.q, p.scale)) / (2 * hh)
        assert abs(fd - dX[t, r]) <= 1e-9 * max(1e-3, abs(dX[t, r])) + 1e-12, (t, r, fd, dX[t, r])
    # tern flips: moving tern[r,c] from a to b changes L by exactly (b - a) * gq[r, c]
    base = L(p.X, p.q, p.scale)
    tern = o.tern(p.q, p.theta)
    for (r, c) in [(0, 0), (4, 9), (19, 31), (10, 16), (7, 2)]:
        for newq in (5, 0, -5):
            q2 = p.q.copy()
            q2[r, c] = newq
            b = {5: 1, 0: 0, -5: -1}[newq]
            d = L(p.X, q2, p.scale) - base
            want = (b - int(tern[r, c])) * gq[r, c]
            assert abs(d - want) <= 1e-10 * max(1.0, abs(base)), (r, c, newq, d, want)


def pin_dead_zone(o):
    """theta above every |q|: tern = 0, so Y, dX and sgrad vanish exactly while
    gq = G * scale is unaffected."""
    p = synth.make_inputs(16, 24, 32, act="bf16", config_id=90)
    Y = o.linear_fwd(p.X, p.q, 8, p.scale)
    dX = o.linear_dx(p.dY, p.q, 8, p.scale)
    G, gq, sg = o.linear_wgrad(p.X, p.dY, p.q, 8, p.scale, want_G=True)
    assert np.all(Y == 0) and np.all(dX == 0) and np.all(sg == 0)
    X = o.widen(p.X)
    dY = o.widen(p.dY)
    assert _rel(G, X.T @ dY) < 1e-13
    assert _rel(gq, (X.T @ dY) * p.scale.astype(np.float64)[None, :]) < 1e-13


def pin_sampling_consistent(o):
    """Sampled rows / columns equal the corresponding full results bit for bit."""
    p = synth.make_inputs(40, 24, 48, act="bf16", config_id=91)
    rows = np.array([0, 7, 39, 13], dtype=np.int64)
    cols = np.array([47, 0, 16, 5], dtype=np.int64)
    Y = o.linear_fwd(p.X, p.q, 2, p.scale)
    dX = o.linear_dx(p.dY, p.q, 2, p.scale)
    G, gq, sg = o.linear_wgrad(p.X, p.dY, p.q, 2, p.scale, want_G=True)
    assert np.array_equal(o.linear_fwd(p.X, p.q, 2, p.scale, rows=rows), Y[rows])
    assert np.array_equal(o.linear_dx(p.dY, p.q, 2, p.scale, rows=rows), dX[rows])
    G2, gq2, sg2 = o.linear_wgrad(p.X, p.dY, p.q, 2, p.scale, cols=cols, want_G=True)
    assert np.array_equal(G2, G[:, cols])
    assert np.array_equal(gq2, gq[:, cols])
    assert np.array_equal(sg2, sg[cols])


def pin_widen(o):
    """bf16 widening is exact: bits 0x3F80 = 1, 0xC000 = -2, 0x0001 = the
    smallest subnormal 2^-133, 0x7F7F = the largest finite bf16."""
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x0000, 0x8000, 0x4049], dtype=np.uint16)
    want = [1.0, -2.0, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127, 0.0, -0.0, 3.140625]
    got = o.widen(bits)
    assert list(got) == want, list(got)


def pin_panel_golden(o):
    """The SR4 health panel of a hand-counted 2 x 8 example
    (tests/golden/panel_example.txt)."""
    g = _golden_kv("panel_example.txt")
    q = np.array([[int(v) for v in g["q0"][0]], [int(v) for v in g["q1"][0]]], dtype=np.int8)
    scale = np.array([float(v) for v in g["scale"][0]], dtype=np.float32)
    r = o.panel([(q, np.zeros_like(q), scale)], int(g["theta"][0][0]), int(g["clamp"][0][0]))
    for k in ("total", "neg", "zero", "pos", "rail", "dead", "churn"):
        assert r[k] == int(g[k][0][0]), (k, r[k])
    for k in ("scale_sum", "scale_mean", "scale_min", "scale_max"):
        assert r[k] == float(g[k][0][0]), (k, r[k])
    assert r["churn_frac"] == 10 / 16 and r["rail_pct"] == 4 / 16


def _panel_brute(mats, theta, clamp):
    """Counts written out independently in pure Python."""
    c = dict(total=0, neg=0, zero=0, pos=0, rail=0, dead=0, churn=0)
    svals = []
    for q, prev, scale in mats:
        for k, v in enumerate(q.reshape(-1).tolist()):
            t = 1 if v >= theta else (-1 if v <= -theta else 0)
            c["total"] += 1
            c["neg" if t < 0 else ("pos" if t > 0 else "zero")] += 1
            c["rail"] += abs(v) == clamp
            c["dead"] += abs(v) < theta
            if prev is not None:
                c["churn"] += int(prev.reshape(-1)[k]) != t
        svals += [float(x) for x in scale]
    return c, svals


def pin_panel_brute_and_invariants(o):
    """Panel counts equal pure-Python counting over several matrices, and the
    definitions' invariants hold: zero == dead (a zero ternary value is exactly
    |q| < theta), neg + zero + pos == total, churn 0 against the matrix's own
    classification and neg + pos against its negation."""
    rng = np.random.default_rng(5)
    for theta, clamp in ((2, 7), (1, 7), (3, 5)):
        mats = []
        for shape in ((3, 16), (5, 24), (1, 8)):
            q = rng.integers(-9, 10, size=shape).astype(np.int8)
            q.reshape(-1)[0] = clamp
            q.reshape(-1)[-1] = -128
            prev = rng.integers(-1, 2, size=shape).astype(np.int8)
            scale = rng.uniform(0.01, 0.1, size=shape[1]).astype(np.float32)
            mats.append((q, prev, scale))
        r = o.panel(mats, theta, clamp)
        want, svals = _panel_brute(mats, theta, clamp)
        for k, v in want.items():
            assert r[k] == v, (theta, clamp, k, r[k], v)
        assert r["scale_count"] == len(svals)
        assert r["scale_min"] == min(svals) and r["scale_max"] == max(svals)
        assert abs(r["scale_sum"] - sum(svals)) <= 1e-12 * len(svals)
        assert r["zero"] == r["dead"] and r["neg"] + r["zero"] + r["pos"] == r["total"]
        own = [(q, o.tern(q, theta), s) for q, _, s in mats]
        assert o.panel(own, theta, clamp)["churn"] == 0
        neg = [(q, -o.tern(q, theta), s) for q, _, s in mats]
        rn = o.panel(neg, theta, clamp)
        assert rn["churn"] == rn["neg"] + rn["pos"]
        # without a previous classification for every matrix there is no churn
        assert o.panel([mats[0], (mats[1][0], None, mats[1][2])], theta, clamp)["churn_frac"] == 0.0


def pin_adamw_closed_forms(o):
    """AdamW on the scale, pinned by closed forms of the textbook update:
    * a constant gradient from zero moments gives m = g (1 - b1^t) exactly, so
      the bias-corrected moments are g and g^2 and every step moves the scale
      by lr g / (|g| + eps) (a zero gradient does not move it);
    * with zero gradient and weight decay, scale_t = scale_0 (1 - lr wd)^t;
    * the page's factor scale_lr / lr multiplies the gradient: after one step
      from zero, m = (1 - b1) g scale_lr / lr;
    * without eps the step does not depend on that factor (Adam's invariance
      to a constant gradient scale)."""
    rng = np.random.default_rng(7)
    g = np.concatenate([rng.normal(0.0, 3e-2, 12), [0.0, 1e-9, -4.0]])
    n = g.size
    s0 = rng.uniform(0.01, 0.1, n)
    lr, b1, b2, eps = 2e-3, 0.9, 0.999, 1e-8
    s, m, v = s0.copy(), np.zeros(n), np.zeros(n)
    for t in range(1, 21):
        s, m, v = o.scale_adamw(g, s, m, v, t, lr, lr, b1, b2, eps, 0.0)
        assert np.allclose(m, g * (1.0 - b1 ** t), rtol=1e-12, atol=0.0), t
        assert np.allclose(v, g * g * (1.0 - b2 ** t), rtol=1e-12, atol=0.0), t
        want = s0 - t * lr * g / (np.abs(g) + eps)
        assert np.allclose(s, want, rtol=1e-12, atol=1e-15), t
    wd = 0.1
    s, m, v = s0.copy(), np.zeros(n), np.zeros(n)
    for t in range(1, 6):
        s, m, v = o.scale_adamw(np.zeros(n), s, m, v, t, lr, lr, b1, b2, eps, wd)
    assert np.allclose(s, s0 * (1.0 - lr * wd) ** 5, rtol=1e-13, atol=0.0)
    _, m1, _ = o.scale_adamw(g, s0, np.zeros(n), np.zeros(n), 1, lr, 10.0 * lr, b1, b2, eps, 0.0)
    assert np.allclose(m1, (1.0 - b1) * g * 10.0, rtol=1e-13, atol=0.0)
    m0 = rng.normal(0.0, 1e-2, n)
    v0 = rng.uniform(1e-5, 1e-3, n)
    a, _, _ = o.scale_adamw(g, s0, m0 * 10.0, v0 * 100.0, 3, lr, 10.0 * lr, b1, b2, 0.0, 0.0)
    b, _, _ = o.scale_adamw(g, s0, m0, v0, 3, lr, lr, b1, b2, 0.0, 0.0)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-16)


ALL_PINS = [pin_tern_golden, pin_tern_properties, pin_pack_golden, pin_pack_roundtrip,
            pin_worked_example, pin_brute_force, pin_sign_matrix_gemm,
            pin_bilinear_identities, pin_finite_differences, pin_dead_zone,
            pin_sampling_consistent, pin_widen, pin_panel_golden, pin_panel_brute_and_invariants,
            pin_adamw_closed_forms]
