"""Parity of the HIP path (through the C ABI) with the CPU oracle on the GPU.

Gates: packing bit-exact; Y, dX, gq and sgrad within rel-L2 2e-3 for bf16
activations and 1e-5 for fp32.  Small shapes are compared element by element
in full; the benchmark workloads at full size are compared on seeded samples
of token rows (Y, dX) and output columns (gq, sgrad) that the oracle computes
one by one, in the same launch configuration the benchmark uses.
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
    tl.lib()  # raises if the HIP library is not built
    yield
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def o():
    return oracle.get()


def check_full(o, p, res, tag):
    tol = tol_for(p.act)
    want = dict(Y=o.linear_fwd(p.X, p.q, p.theta, p.scale),
                dX=o.linear_dx(p.dY, p.q, p.theta, p.scale))
    _, want["gq"], want["sgrad"] = o.linear_wgrad(p.X, p.dY, p.q, p.theta, p.scale)
    want_pk = o.pack(o.tern(p.q, p.theta))
    assert np.array_equal(res["packed"], want_pk), f"{tag}: packing differs"
    errs = {k: rel_l2(res[k], want[k]) for k in ("Y", "dX", "gq", "sgrad")}
    log(f"  {tag}: relL2 {errs}")
    for k, e in errs.items():
        assert e <= tol, f"{tag}: {k} relL2 {e:.3e} > {tol:.1e}"
    check_elements(o, p, res, want, tag=tag)
    return errs


# ---------------------------------------------------------------------------
# materialize: bit-exact packing
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("theta", [1, 2, 3, 7, 8, 127])
def test_materialize_all_int8(o, theta):
    log(f"materialize all int8 values theta={theta}")
    q = ((np.arange(256 * 64).reshape(256, 64) % 256) - 128).astype(np.int8)
    qd = to_dev(q)
    pk = tl.empty_packed(256, 64)
    tl.tern_materialize(qd, theta, pk)
    torch.cuda.synchronize()
    got = tl.packed_canonical(pk, 256, 64).cpu().numpy().view(np.uint32)
    assert np.array_equal(got, o.pack(o.tern(q, theta)))


@pytest.mark.parametrize("n_in,n_out", [(1, 8), (3, 24), (37, 40), (5, 72), (64, 1000), (17, 16), (9, 4096)])
@pytest.mark.parametrize("aligned", [True, False])
def test_materialize_ragged(o, n_in, n_out, aligned):
    log(f"materialize ragged in={n_in} out={n_out} aligned={aligned}")
    q = synth.int8_uniform(synth.stream_seed(5, n_in, n_out, 0), (n_in, n_out), -128, 127)
    flat = torch.zeros(n_in * n_out + 16, dtype=torch.int8, device="cuda")
    off = 0 if aligned else 3
    qd = flat[off:off + n_in * n_out].view(n_in, n_out)
    qd.copy_(to_dev(q))
    pk = tl.empty_packed(n_in, n_out)
    for theta in (2, 5):
        tl.tern_materialize(qd, theta, pk)
        torch.cuda.synchronize()
        got = tl.packed_canonical(pk, n_in, n_out).cpu().numpy().view(np.uint32)
        assert np.array_equal(got, o.pack(o.tern(q, theta)))


# ---------------------------------------------------------------------------
# full element-by-element parity on small and ragged shapes
# ---------------------------------------------------------------------------

SMALL = [(1, 8, 8), (3, 8, 16), (5, 24, 40), (64, 64, 64), (70, 24, 40), (129, 72, 136),
         (257, 136, 264), (300, 200, 520), (1000, 64, 1024), (96, 1024, 64), (2, 2048, 16),
         (517, 512, 264)]


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("T,n_in,n_out", SMALL)
def test_parity_small(o, T, n_in, n_out, act):
    log(f"parity small T={T} in={n_in} out={n_out} act={act}")
    p = synth.make_inputs(T, n_in, n_out, act=act, config_id=200 + T % 97, proj_id=n_in + n_out)
    d = DeviceProjection(p)
    d.step()
    check_full(o, p, d.results(), f"T={T} in={n_in} out={n_out} {act}")


@pytest.mark.parametrize("q_law,scale_law,theta", [("skewed", "lognormal", 2), ("uniform", "uniform", 1),
                                                   ("uniform", "lognormal", 6)])
def test_parity_laws(o, q_law, scale_law, theta):
    log(f"parity laws {q_law} {scale_law} theta={theta}")
    p = synth.make_inputs(384, 320, 192, act="bf16", q_law=q_law, scale_law=scale_law, theta=theta,
                          config_id=301)
    d = DeviceProjection(p)
    d.step()
    check_full(o, p, d.results(), f"{q_law}/{scale_law}/theta={theta}")


def test_parity_tiny_config(o):
    w = synth.WORKLOADS["tiny"]
    log("parity tiny workload (fp32)")
    p = synth.workload_inputs(w, 0)
    d = DeviceProjection(p)
    d.step()
    check_full(o, p, d.results(), "tiny")


@pytest.mark.parametrize("proj", range(6))
def test_parity_rwkv_small_full(o, proj):
    w = synth.WORKLOADS["rwkv_small"]
    log(f"parity rwkv_small projection {w.projs[proj]} (full)")
    p = synth.workload_inputs(w, proj)
    d = DeviceProjection(p)
    d.step()
    check_full(o, p, d.results(), f"rwkv_small/{w.projs[proj][0]}")


# Shapes that the planner serves with 128-row tiles (the first) and with the
# persistent 256-row tiles (the other two: dW split in four, and unsplit) in
# all three products, for both activation types, ragged in every dimension
# (1000 = 7*128 + 104, 1032 = 4*256 + 8, 4000 = 15*256 + 160, 2056 = 8*256 + 8),
# compared element by element.
@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("T,n_in,n_out", [(1000, 1032, 1032), (4000, 1032, 1032), (2056, 2056, 2056)])
def test_parity_big_tiles_full(o, T, n_in, n_out, act):
    log(f"parity big tiles (full) T={T} in={n_in} out={n_out} act={act}")
    p = synth.make_inputs(T, n_in, n_out, act=act, config_id=870, proj_id=T + n_in)
    d = DeviceProjection(p)
    d.step()
    check_full(o, p, d.results(), f"T={T} in={n_in} out={n_out} {act}")


def test_y_bf16_output(o):
    log("forward with bf16 Y")
    p = synth.make_inputs(260, 136, 520, act="bf16", config_id=302)
    d = DeviceProjection(p, y_bf16=True)
    d.materialize()
    d.fwd()
    torch.cuda.synchronize()
    Yb = d.Y.float().cpu().numpy()
    Y = o.linear_fwd(p.X, p.q, p.theta, p.scale)
    assert rel_l2(Yb, Y) <= 2e-3
    # the bf16 output is the round-to-nearest-even of the fp32 output
    Yf = torch.empty((p.X.shape[0], 520), dtype=torch.float32, device="cuda")
    tl.tern_linear_fwd(d.X, d.packed, d.scale, Yf)
    torch.cuda.synchronize()
    assert torch.equal(Yf.to(torch.bfloat16).float().cpu(), torch.from_numpy(Yb))


# ---------------------------------------------------------------------------
# exact-arithmetic regime: every partial sum is an exact fp32 integer multiple
# of the scale's power of two, so any summation order gives the same bits
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("T,n_in,n_out", [(64, 64, 64), (300, 200, 520), (1000, 256, 264)])
def test_exact_regime_bitwise(o, T, n_in, n_out, act):
    log(f"exact regime T={T} in={n_in} out={n_out} {act}")
    base = synth.make_inputs(T, n_in, n_out, act="f32", config_id=400 + n_in)
    Xi = synth.int8_uniform(synth.stream_seed(11, T, n_in, 0), (T, n_in), -3, 3).astype(np.float32)
    dYi = synth.int8_uniform(synth.stream_seed(11, T, n_out, 1), (T, n_out), -3, 3).astype(np.float32)
    k = synth.int8_uniform(synth.stream_seed(11, n_out, 0, 2), (n_out,), 2, 9).astype(np.float32)
    scale = (2.0 ** -k).astype(np.float32)
    if act == "bf16":
        Xi, dYi = synth.to_bf16_bits(Xi), synth.to_bf16_bits(dYi)
    p = synth.ProjInputs(Xi, dYi, base.q, scale, 2, act)
    d = DeviceProjection(p)
    d.step()
    r = d.results()
    Y = o.linear_fwd(p.X, p.q, 2, p.scale)
    dX = o.linear_dx(p.dY, p.q, 2, p.scale)
    _, gq, sg = o.linear_wgrad(p.X, p.dY, p.q, 2, p.scale)
    assert np.array_equal(r["Y"].astype(np.float64), Y)
    assert np.array_equal(r["dX"].astype(np.float64), dX)
    assert np.array_equal(r["gq"].astype(np.float64), gq)
    assert np.array_equal(r["sgrad"].astype(np.float64), sg)


# ---------------------------------------------------------------------------
# the benchmark workloads at full size, sampled
# ---------------------------------------------------------------------------

def sampled_case(o, wname, proj):
    w = synth.WORKLOADS[wname]
    name, n_in, n_out = w.projs[proj]
    log(f"parity {wname}/{name} T={w.T} in={n_in} out={n_out} (full size, sampled)")
    p = synth.workload_inputs(w, proj)
    d = DeviceProjection(p)
    d.step()
    torch.cuda.synchronize()
    rows = np.union1d(synth.sample_indices(synth.stream_seed(77, w.config_id, proj, 0), 40, w.T),
                      [0, w.T - 1])
    cols = np.union1d(synth.sample_indices(synth.stream_seed(77, w.config_id, proj, 1), 14, n_out),
                      [0, n_out - 1])
    rt = torch.from_numpy(rows).cuda()
    ct = torch.from_numpy(cols).cuda()
    Yg = d.Y[rt].cpu().numpy()
    dXg = d.dX[rt].cpu().numpy()
    gqg = d.gq[:, ct].cpu().numpy()
    sgg = d.sgrad[ct].cpu().numpy()
    pk = tl.packed_canonical(d.packed, n_in, n_out).cpu().numpy().view(np.uint32)
    assert np.array_equal(pk, o.pack(o.tern(p.q, p.theta))), "packing differs"
    want = dict(Y=o.linear_fwd(p.X, p.q, p.theta, p.scale, rows=rows),
                dX=o.linear_dx(p.dY, p.q, p.theta, p.scale, rows=rows))
    _, want["gq"], want["sgrad"] = o.linear_wgrad(p.X, p.dY, p.q, p.theta, p.scale, cols=cols)
    got = dict(Y=Yg, dX=dXg, gq=gqg, sgrad=sgg)
    errs = {k: rel_l2(got[k], want[k]) for k in got}
    log(f"  relL2 {errs}")
    tol = tol_for(p.act)
    for k, e in errs.items():
        assert e <= tol, f"{wname}/{name}: {k} relL2 {e:.3e} > {tol:.1e}"
    check_elements(o, p, got, want, rows=rows, cols=cols, tag=f"{wname}/{name}")


# Shapes on which every product takes the persistent kernels with ragged edges:
# M and N off the tile grid, K off the 32-wide chunk grid with an odd chunk
# count (the padding chunk), and a token count off the 64-token dW chunk.
@pytest.mark.parametrize("T,n_in,n_out", [(4000, 1032, 4104), (4000, 4104, 1032)])
def test_parity_tile256_ragged_sampled(o, T, n_in, n_out):
    log(f"parity 256-tile kernels, ragged T={T} in={n_in} out={n_out} (sampled)")
    p = synth.make_inputs(T, n_in, n_out, act="bf16", config_id=303, proj_id=n_in)
    d = DeviceProjection(p)
    d.step()
    torch.cuda.synchronize()
    rows = np.union1d(synth.sample_indices(synth.stream_seed(78, T, n_in, 0), 40, T), [0, T - 1])
    cols = np.union1d(synth.sample_indices(synth.stream_seed(78, T, n_out, 1), 14, n_out), [0, n_out - 1])
    rt = torch.from_numpy(rows).cuda()
    ct = torch.from_numpy(cols).cuda()
    want = dict(Y=o.linear_fwd(p.X, p.q, p.theta, p.scale, rows=rows),
                dX=o.linear_dx(p.dY, p.q, p.theta, p.scale, rows=rows))
    _, want["gq"], want["sgrad"] = o.linear_wgrad(p.X, p.dY, p.q, p.theta, p.scale, cols=cols)
    got = dict(Y=d.Y[rt].cpu().numpy(), dX=d.dX[rt].cpu().numpy(), gq=d.gq[:, ct].cpu().numpy(),
               sgrad=d.sgrad[ct].cpu().numpy())
    errs = {k: rel_l2(got[k], want[k]) for k in got}
    log(f"  relL2 {errs}")
    for k, e in errs.items():
        assert e <= tol_for("bf16"), f"{k} relL2 {e:.3e}"
    check_elements(o, p, got, want, rows=rows, cols=cols, tag=f"T={T} in={n_in} out={n_out}")
    # bf16 Y from the same kernel is the round-to-nearest-even of its fp32 Y
    Yb = torch.empty((T, n_out), dtype=torch.bfloat16, device="cuda")
    tl.tern_linear_fwd(d.X, d.packed, d.scale, Yb)
    torch.cuda.synchronize()
    assert torch.equal(Yb, d.Y.to(torch.bfloat16))


@pytest.mark.parametrize("proj", range(6))
def test_parity_mid_sampled(o, proj):
    sampled_case(o, "mid", proj)


@pytest.mark.parametrize("proj", range(6))
def test_parity_large_sampled(o, proj):
    sampled_case(o, "large", proj)


@pytest.mark.parametrize("proj", [0, 4, 5])
def test_parity_largest_sampled(o, proj):
    sampled_case(o, "largest", proj)


def test_parity_operands_beyond_4gib(o):
    """X of 4 GiB (T = 262144 tokens x 8192 bf16) and dX of 8 GiB: tile base
    offsets far past 2^32 bytes, through the same kernels as the benchmark
    (the 512 x 128 forward / dX and the split-K 256 x 256 dW); sampled rows and columns
    against the oracle."""
    T, n_in, n_out = 262144, 8192, 256
    log(f"parity beyond 4 GiB: T={T} in={n_in} out={n_out}")
    p = synth.make_inputs(T, n_in, n_out, act="bf16", config_id=305)
    d = DeviceProjection(p)
    d.step()
    torch.cuda.synchronize()
    rows = np.union1d(synth.sample_indices(synth.stream_seed(83, T, n_in, 0), 24, T), [0, T // 2, T - 1])
    cols = np.union1d(synth.sample_indices(synth.stream_seed(83, T, n_out, 1), 3, n_out), [n_out - 1])
    rt, ct = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    want = dict(Y=o.linear_fwd(p.X, p.q, p.theta, p.scale, rows=rows),
                dX=o.linear_dx(p.dY, p.q, p.theta, p.scale, rows=rows))
    _, want["gq"], want["sgrad"] = o.linear_wgrad(p.X, p.dY, p.q, p.theta, p.scale, cols=cols)
    got = dict(Y=d.Y[rt].cpu().numpy(), dX=d.dX[rt].cpu().numpy(), gq=d.gq[:, ct].cpu().numpy(),
               sgrad=d.sgrad[ct].cpu().numpy())
    errs = {k: rel_l2(got[k], want[k]) for k in got}
    log(f"  relL2 {errs}")
    for k, e in errs.items():
        assert e <= tol_for("bf16"), f"{k} relL2 {e:.3e}"
    check_elements(o, p, got, want, rows=rows, cols=cols, tag=f"T={T} in={n_in} out={n_out}")
    pk = tl.packed_canonical(d.packed, n_in, n_out).cpu().numpy().view(np.uint32)
    assert np.array_equal(pk, o.pack(o.tern(p.q, p.theta))), "packing differs"


def _frag_copy(tern, M_is_in):
    """The fragment-ordered copy of include/tern.h, built from a tern matrix
    [in, out] of {-1, 0, 1}: operand A[m][k] = tern[k][m] (forward copy,
    M_is_in False) or tern[m][k] (dX copy).  Word (tile, chunk, wm, lane, fm)
    holds the values of row m = 256 tile + 128 wm + 32 fm + lane % 32 at
    k = 32 chunk + 16 kk + 8 (lane // 32) + e in nibble e: for kk = 0 the
    fp4 (e2m1) encoding of the value (+1 = 0x2, -1 = 0xA, 0 = 0x0), for
    kk = 1 the same shifted right by one bit."""
    A = tern if M_is_in else tern.T
    M, K = A.shape
    tiles, nch = -(-M // 256), -(-K // 32)
    Ap = np.zeros((tiles * 256, nch * 32), np.int64)
    Ap[:M, :K] = A
    fp4 = np.where(Ap > 0, 0x2, np.where(Ap < 0, 0xA, 0)).astype(np.uint64)
    c = fp4.reshape(tiles, 2, 4, 32, nch, 2, 2, 8)         # tile, wm, fm, l32, chunk, kk, h, e
    c = c.transpose(0, 4, 1, 6, 3, 2, 5, 7)                # tile, chunk, wm, h, l32, fm, kk, e
    c = c >> np.arange(2, dtype=np.uint64)[:, None]        # kk = 1 one bit lower
    pos = 4 * np.arange(8, dtype=np.uint64)[None, :]
    word = (c << pos).sum(axis=(-2, -1))                   # values occupy disjoint bits
    return word.reshape(-1).astype(np.uint32)


@pytest.mark.parametrize("n_in,n_out", [(8, 8), (136, 264), (520, 776), (264, 1032)])
def test_fragment_copies(o, n_in, n_out):
    """The handle's two fragment-ordered copies hold exactly the codes of the
    canonical matrix, in the documented order (edges padded with 00)."""
    log(f"fragment copies in={n_in} out={n_out}")
    q = synth.int8_uniform(synth.stream_seed(6, n_in, n_out, 0), (n_in, n_out), -7, 7)
    pk = tl.empty_packed(n_in, n_out)
    tl.tern_materialize(to_dev(q), 2, pk)
    torch.cuda.synchronize()
    got = pk.cpu().numpy().view(np.uint32)
    t = o.tern(q, 2)
    canon = n_in * (-(-n_out // 16))
    fwd_off = -(-canon // 64) * 64
    fwd = _frag_copy(t, False)
    dxc = _frag_copy(t, True)
    assert got.size == fwd_off + fwd.size + dxc.size
    assert np.array_equal(got[fwd_off:fwd_off + fwd.size], fwd), "forward copy differs"
    assert np.array_equal(got[fwd_off + fwd.size:], dxc), "dX copy differs"


@pytest.mark.parametrize("n_in,n_out", [(264, 520), (3, 24), (136, 1032)])
def test_materialize_writes_every_word(n_in, n_out):
    """Every word of the handle is written, the alignment padding between the
    canonical matrix and the copies included: handles that start as all-zero
    and all-one bits end up identical."""
    log(f"materialize fills the handle in={n_in} out={n_out}")
    q = to_dev(synth.int8_uniform(synth.stream_seed(7, n_in, n_out, 0), (n_in, n_out), -7, 7))
    a = tl.empty_packed(n_in, n_out)
    b = tl.empty_packed(n_in, n_out)
    a.fill_(0)
    b.fill_(-1)
    tl.tern_materialize(q, 2, a)
    tl.tern_materialize(q, 2, b)
    torch.cuda.synchronize()
    assert torch.equal(a, b), "some handle words keep their previous contents"


# ---------------------------------------------------------------------------
# properties
# ---------------------------------------------------------------------------

def test_bwd_deterministic_and_split_equal():
    log("determinism: repeated bwd and bwd_dx + bwd_dw")
    for (T, n_in, n_out) in [(4096, 512, 2048), (2048, 1024, 1024), (777, 264, 136)]:
        p = synth.make_inputs(T, n_in, n_out, act="bf16", config_id=500)
        d = DeviceProjection(p)
        d.step()
        r1 = d.results()
        d.bwd()
        d.fwd()
        r2 = d.results()
        for k in ("Y", "dX", "gq", "sgrad"):
            assert np.array_equal(r1[k], r2[k]), f"{k} differs between identical calls"
        dX = torch.empty_like(d.dX)
        gq = torch.empty_like(d.gq)
        sg = torch.empty_like(d.sgrad)
        tl.tern_linear_bwd_dx(d.dY, d.packed, d.scale, dX)
        tl.tern_linear_bwd_dw(d.X, d.dY, d.packed, d.scale, gq, sg, d.ws)
        torch.cuda.synchronize()
        assert torch.equal(dX, d.dX) and torch.equal(gq, d.gq) and torch.equal(sg, d.sgrad)


def test_zero_sizes():
    log("zero sizes")
    dev = "cuda"
    # T = 0: G is an empty sum, so gq = 0 and sgrad = 0
    X = torch.empty((0, 64), dtype=torch.bfloat16, device=dev)
    dY = torch.empty((0, 32), dtype=torch.bfloat16, device=dev)
    q = torch.ones((64, 32), dtype=torch.int8, device=dev) * 3
    sc = torch.ones(32, device=dev)
    pk = tl.empty_packed(64, 32)
    tl.tern_materialize(q, 2, pk)
    Y = torch.empty((0, 32), device=dev)
    tl.tern_linear_fwd(X, pk, sc, Y)
    dX = torch.empty((0, 64), device=dev)
    gq = torch.full((64, 32), 7.0, device=dev)
    sg = torch.full((32,), 7.0, device=dev)
    ws = tl.empty_workspace(0, 64, 32)
    tl.tern_linear_bwd(X, dY, pk, sc, dX, gq, sg, ws)
    torch.cuda.synchronize()
    assert torch.all(gq == 0) and torch.all(sg == 0)
    # in = 0: Y = 0 (empty sum over r), sgrad = 0
    X = torch.empty((16, 0), dtype=torch.bfloat16, device=dev)
    dY = torch.randn((16, 32), device=dev).to(torch.bfloat16)
    pk = tl.empty_packed(0, 32)
    Y = torch.full((16, 32), 7.0, device=dev)
    tl.tern_linear_fwd(X, pk, sc, Y)
    dX = torch.empty((16, 0), device=dev)
    gq = torch.empty((0, 32), device=dev)
    sg = torch.full((32,), 7.0, device=dev)
    tl.tern_linear_bwd(X, dY, pk, sc, dX, gq, sg, tl.empty_workspace(16, 0, 32))
    torch.cuda.synchronize()
    assert torch.all(Y == 0) and torch.all(sg == 0)
    # out = 0: dX = 0 (empty sum over c)
    X = torch.randn((16, 24), device=dev).to(torch.bfloat16)
    dY = torch.empty((16, 0), dtype=torch.bfloat16, device=dev)
    pk = tl.empty_packed(24, 0)
    sc0 = torch.empty((0,), device=dev)
    dX = torch.full((16, 24), 7.0, device=dev)
    gq = torch.empty((24, 0), device=dev)
    sg = torch.empty((0,), device=dev)
    Y = torch.empty((16, 0), device=dev)
    tl.tern_linear_fwd(X, pk, sc0, Y)
    tl.tern_linear_bwd(X, dY, pk, sc0, dX, gq, sg, tl.empty_workspace(16, 24, 0))
    torch.cuda.synchronize()
    assert torch.all(dX == 0)


def test_outputs_stay_in_bounds():
    """Guard bytes around every output are untouched (ragged shapes)."""
    log("canaries around outputs")
    T, n_in, n_out = 333, 200, 136
    p = synth.make_inputs(T, n_in, n_out, act="bf16", config_id=600)
    d = DeviceProjection(p)
    G = 4096  # guard elements on each side

    def guarded(shape, dtype):
        n = int(np.prod(shape))
        buf = torch.full((n + 2 * G,), 1234.5, dtype=dtype, device="cuda")
        return buf, buf[G:G + n].view(shape)

    bY, Y = guarded((T, n_out), torch.float32)
    bX, dX = guarded((T, n_in), torch.float32)
    bq, gq = guarded((n_in, n_out), torch.float32)
    bs, sg = guarded((n_out,), torch.float32)
    npk = tl.tern_packed_words(n_in, n_out)
    bp = torch.full((npk + 2 * G,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    pk = bp[G:G + npk]
    tl.tern_materialize(d.q, 2, pk)
    tl.tern_linear_fwd(d.X, pk, d.scale, Y)
    tl.tern_linear_bwd(d.X, d.dY, pk, d.scale, dX, gq, sg, d.ws)
    torch.cuda.synchronize()
    for b in (bY, bX, bq, bs):
        assert torch.all(b[:G] == 1234.5) and torch.all(b[-G:] == 1234.5)
    assert torch.all(bp[:G] == 0x5A5A5A5A) and torch.all(bp[-G:] == 0x5A5A5A5A)
