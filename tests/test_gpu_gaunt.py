"""GPU parity of the Gaunt (spherical-grid) convolution against the float64
oracle, which sums Gaunt coefficients over per-edge messages.  Every output
degree block within 1e-4 of max|ref| of that block; repeated runs bitwise
equal; isolated receivers and an empty graph give zeros."""
import numpy as np
import pytest

import oracle
from tests.test_gpu_parity import T, block_err, say
from workloads import make_gaunt_weights, make_workload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 1e-4


@pytest.fixture(scope="module")
def tpc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tensor_product_convolution_amd as m
    m.lib()
    return m


def _case(irr, lsh, lout, graph, n, seed=0):
    gp = oracle.gaunt_plan(irr, lsh, lout)
    dims = dict(xdim=gp.xdim, n_paths=1, U=gp.U, outdim=gp.outdim, n_out_irreps=lout + 1)
    wl = make_workload("mid", dims, seed=seed, n_nodes=n)
    if graph != "mid":
        gw = make_workload(graph, dims, seed=seed, n_nodes=n, graph_only=True)
        wl.src, wl.dst, wl.r = gw.src, gw.dst, gw.r
    w = make_gaunt_weights(wl.n_edges, lsh, gp.U, seed)
    return gp, wl, w


def _blocks(gp):
    return [slice(gp.out_offsets[l], gp.out_offsets[l] + gp.U * (2 * l + 1))
            for l in range(gp.lmax_out + 1)]


def _gpu(tpc, irr, lsh, lout, wl, w):
    plan = tpc.Plan(irr, lsh, lout, mode=tpc.TP_MODE_GAUNT)
    g = tpc.graph_build(T(wl.src), T(wl.dst), wl.n_nodes)
    Y = tpc.sph_harm(lsh, tpc.gather_rows(T(wl.r), g.perm))
    ws = tpc.gather_rows(T(w.reshape(w.shape[0], w.shape[1] * w.shape[2])), g.perm)
    out = tpc.forward_gaunt(plan, g, T(wl.x), Y, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _ref(gp, wl, w):
    return oracle.gaunt_conv_fwd(gp, wl.src, wl.dst, wl.n_nodes, wl.x,
                                 oracle.sh_real(gp.lmax_sh, wl.r), w)


@pytest.mark.parametrize("U,irr_t,lsh,lout,graph,n", [
    (16, "{U}x0e+{U}x1o+{U}x2e", 2, 2, "tiny", 32),
    (32, "{U}x0e+{U}x1o+{U}x2e", 2, 2, "mid", 300),
    (32, "{U}x0e+{U}x1o+{U}x2e", 2, 2, "zipf", 400),
    (64, "{U}x0e+{U}x1o+{U}x2e", 2, 2, "lmax3", 200),
    (128, "{U}x0e+{U}x1o+{U}x2e", 2, 2, "mid", 120),
    (32, "{U}x1o+{U}x0e", 1, 2, "mid", 150),
    (16, "{U}x2e", 1, 1, "mid", 150),
    (32, "{U}x0e+{U}x1o+{U}x2e", 2, 2, "mid", 1536),
])
def test_gaunt_forward_parity(tpc, U, irr_t, lsh, lout, graph, n):
    irr = irr_t.format(U=U)
    say(f"gaunt forward {irr} lsh={lsh} lout={lout} graph={graph} n={n}")
    gp, wl, w = _case(irr, lsh, lout, graph, n)
    got = _gpu(tpc, irr, lsh, lout, wl, w)
    ref = _ref(gp, wl, w)
    assert block_err(got, ref, _blocks(gp)) <= TOL


def test_gaunt_deterministic_isolated_and_empty(tpc):
    say("gaunt forward determinism, isolated nodes, empty graph")
    irr = "32x0e+32x1o+32x2e"
    gp, wl, w = _case(irr, 2, 2, "mid", 90, seed=4)
    keep = wl.dst >= 10
    wl.src, wl.dst, wl.r, w = wl.src[keep], wl.dst[keep], wl.r[keep], w[keep]
    a = _gpu(tpc, irr, 2, 2, wl, w)
    b = _gpu(tpc, irr, 2, 2, wl, w)
    assert np.array_equal(a, b)
    assert np.all(a[:10] == 0)
    assert block_err(a, _ref(gp, wl, w), _blocks(gp)) <= TOL
    wl.src, wl.dst, wl.r = wl.src[:0], wl.dst[:0], wl.r[:0]
    assert np.all(_gpu(tpc, irr, 2, 2, wl, w[:0]) == 0)


def _gpu_bwd(tpc, irr, lsh, lout, wl, w, go, want=("x", "Y", "w")):
    plan = tpc.Plan(irr, lsh, lout, mode=tpc.TP_MODE_GAUNT)
    g = tpc.graph_build(T(wl.src), T(wl.dst), wl.n_nodes)
    Y = tpc.sph_harm(lsh, tpc.gather_rows(T(wl.r), g.perm))
    ws = tpc.gather_rows(T(w.reshape(w.shape[0], w.shape[1] * w.shape[2])), g.perm)
    res = tpc.backward_gaunt(plan, g, T(wl.x), Y, ws, T(go), want=want)
    torch.cuda.synchronize()
    return [None if r is None else r.cpu().numpy() for r in res], g.perm.cpu().numpy()


def _bwd_blocks(gp, E):
    xb = [slice(o, o + gp.U * (2 * l + 1)) for l, o in zip(gp.degrees, gp.in_offsets)]
    yb = [slice(l * l, (l + 1) ** 2) for l in range(gp.lmax_sh + 1)]
    wb = [slice(l * gp.U, (l + 1) * gp.U) for l in range(gp.lmax_sh + 1)]
    return xb, yb, wb


@pytest.mark.parametrize("U,irr_t,lsh,lout,graph,n", [
    (16, "{U}x0e+{U}x1o+{U}x2e", 2, 2, "tiny", 32),
    (32, "{U}x0e+{U}x1o+{U}x2e", 2, 2, "mid", 300),
    (32, "{U}x0e+{U}x1o+{U}x2e", 2, 2, "zipf", 400),
    (64, "{U}x0e+{U}x1o+{U}x2e", 2, 2, "lmax3", 200),
    (128, "{U}x0e+{U}x1o+{U}x2e", 2, 2, "mid", 120),
    (32, "{U}x1o+{U}x0e", 1, 2, "mid", 150),
    (16, "{U}x2e", 1, 1, "mid", 150),
    (32, "{U}x0e+{U}x1o+{U}x2e", 2, 2, "mid", 1536),
])
def test_gaunt_backward_parity(tpc, U, irr_t, lsh, lout, graph, n):
    irr = irr_t.format(U=U)
    say(f"gaunt backward {irr} lsh={lsh} lout={lout} graph={graph} n={n}")
    gp, wl, w = _case(irr, lsh, lout, graph, n)
    go = np.random.default_rng(11).normal(size=(wl.n_nodes, gp.outdim)).astype(np.float32)
    (gx, gY, gw), perm = _gpu_bwd(tpc, irr, lsh, lout, wl, w, go)
    rx, rY, rw = oracle.gaunt_conv_bwd(gp, wl.src, wl.dst, wl.n_nodes, wl.x,
                                       oracle.sh_real(lsh, wl.r), w, go)
    xb, yb, wb = _bwd_blocks(gp, wl.n_edges)
    assert block_err(gx, rx, xb) <= TOL
    assert block_err(gY, rY[perm], yb) <= TOL
    assert block_err(gw, rw.reshape(len(rw), -1)[perm], wb) <= TOL


def test_gaunt_backward_subsets_isolated_empty_deterministic(tpc):
    say("gaunt backward output subsets, isolated nodes, empty graph, determinism")
    irr = "32x0e+32x1o+32x2e"
    gp, wl, w = _case(irr, 2, 2, "mid", 90, seed=5)
    keep = (wl.dst >= 10) & (wl.src >= 5)     # receivers 0..9 and senders 0..4 isolated
    wl.src, wl.dst, wl.r, w = wl.src[keep], wl.dst[keep], wl.r[keep], w[keep]
    go = np.random.default_rng(12).normal(size=(wl.n_nodes, gp.outdim)).astype(np.float32)
    (gx, gY, gw), perm = _gpu_bwd(tpc, irr, 2, 2, wl, w, go)
    (gx2, gY2, gw2), _ = _gpu_bwd(tpc, irr, 2, 2, wl, w, go)
    assert np.array_equal(gx, gx2) and np.array_equal(gY, gY2) and np.array_equal(gw, gw2)
    assert np.all(gx[:5] == 0)
    rx, rY, rw = oracle.gaunt_conv_bwd(gp, wl.src, wl.dst, wl.n_nodes, wl.x, oracle.sh_real(2, wl.r), w, go)
    xb, yb, wb = _bwd_blocks(gp, wl.n_edges)
    (sx, sY, sw), _ = _gpu_bwd(tpc, irr, 2, 2, wl, w, go, want=("w",))
    assert sx is None and sY is None and np.array_equal(sw, gw)
    (sx, sY, sw), _ = _gpu_bwd(tpc, irr, 2, 2, wl, w, go, want=("x", "Y"))
    assert sw is None and np.array_equal(sx, gx) and np.array_equal(sY, gY)
    assert block_err(gx, rx, xb) <= TOL
    wl.src, wl.dst, wl.r = wl.src[:0], wl.dst[:0], wl.r[:0]
    (gx, gY, gw), _ = _gpu_bwd(tpc, irr, 2, 2, wl, w[:0], go)
    assert np.all(gx == 0) and gY.size == 0 and gw.size == 0


def _gpu_dbl(tpc, irr, lsh, lout, wl, w, go, cot, want=("x", "Y", "w", "g")):
    """second-order backward on the GPU; edge cotangents in original order"""
    plan = tpc.Plan(irr, lsh, lout, mode=tpc.TP_MODE_GAUNT)
    g = tpc.graph_build(T(wl.src), T(wl.dst), wl.n_nodes)
    Y = tpc.sph_harm(lsh, tpc.gather_rows(T(wl.r), g.perm))
    flat = lambda a: a.reshape(a.shape[0], int(np.prod(a.shape[1:])))
    ws = tpc.gather_rows(T(flat(w)), g.perm)
    ggx, ggY, ggw = cot
    gath = lambda a: None if a is None else tpc.gather_rows(T(flat(a)), g.perm)
    res = tpc.double_backward_gaunt(plan, g, T(wl.x), Y, ws, T(go), gg_x=None if ggx is None else T(ggx),
                                    gg_Y=gath(ggY), gg_w=gath(ggw), want=want)
    torch.cuda.synchronize()
    return [None if r is None else r.cpu().numpy() for r in res], g.perm.cpu().numpy()


def _check_dbl(gp, wl, w, go, cot, got, perm, lsh):
    ref = oracle.gaunt_conv_double_bwd(gp, wl.src, wl.dst, wl.n_nodes, wl.x, oracle.sh_real(lsh, wl.r), w, go,
                                       *cot)
    xb, yb, wb = _bwd_blocks(gp, wl.n_edges)
    dx, dY, dw, dg = got
    if dx is not None:
        assert block_err(dx, ref[0], xb) <= TOL, "d_x"
    if dY is not None:
        assert block_err(dY, ref[1][perm], yb) <= TOL, "d_Y"
    if dw is not None:
        assert block_err(dw, ref[2].reshape(len(ref[2]), -1)[perm], wb) <= TOL, "d_w"
    if dg is not None:
        assert block_err(dg, ref[3], _blocks(gp)) <= TOL, "d_grad_out"


def _gaunt_cot(gp, wl, w, seed):
    rng = np.random.default_rng(seed)
    f = lambda shape: rng.normal(size=shape).astype(np.float32)
    return [f(wl.x.shape), f((wl.n_edges, gp.ysh)), f(w.shape)]


@pytest.mark.parametrize("U,irr_t,lsh,lout,graph,n", [
    (32, "{U}x0e+{U}x1o+{U}x2e", 2, 2, "mid", 300),
    (16, "{U}x0e+{U}x1o+{U}x2e", 2, 2, "zipf", 400),
    (64, "{U}x1o+{U}x0e", 1, 2, "lmax3", 150),
])
def test_gaunt_double_backward_parity(tpc, U, irr_t, lsh, lout, graph, n):
    irr = irr_t.format(U=U)
    say(f"gaunt double backward {irr} lsh={lsh} lout={lout} graph={graph} n={n}")
    gp, wl, w = _case(irr, lsh, lout, graph, n)
    go = np.random.default_rng(12).normal(size=(wl.n_nodes, gp.outdim)).astype(np.float32)
    cot = _gaunt_cot(gp, wl, w, U + n)
    got, perm = _gpu_dbl(tpc, irr, lsh, lout, wl, w, go, cot)
    _check_dbl(gp, wl, w, go, cot, got, perm, lsh)


def test_gaunt_double_backward_subsets_isolated_empty(tpc):
    """Each cotangent alone, none (zeros), output subsets, determinism,
    isolated nodes and the empty graph."""
    say("gaunt double backward: cotangent and output subsets, degenerate graphs")
    irr = "32x0e+32x1o+32x2e"
    gp, wl, w = _case(irr, 2, 2, "mid", 90, seed=6)
    keep = (wl.dst >= 10) & (wl.src >= 5)
    wl.src, wl.dst, wl.r = wl.src[keep], wl.dst[keep], wl.r[keep]
    w = w[keep]
    go = np.random.default_rng(13).normal(size=(wl.n_nodes, gp.outdim)).astype(np.float32)
    cot = _gaunt_cot(gp, wl, w, 51)
    for k in range(3):
        one = [c if i == k else None for i, c in enumerate(cot)]
        got, perm = _gpu_dbl(tpc, irr, 2, 2, wl, w, go, one)
        _check_dbl(gp, wl, w, go, one, got, perm, 2)
    none, _ = _gpu_dbl(tpc, irr, 2, 2, wl, w, go, [None] * 3)
    assert all(np.all(a == 0) for a in none)
    full, perm = _gpu_dbl(tpc, irr, 2, 2, wl, w, go, cot)
    _check_dbl(gp, wl, w, go, cot, full, perm, 2)
    assert np.all(full[0][:5] == 0) and np.all(full[3][:10] == 0)
    again, _ = _gpu_dbl(tpc, irr, 2, 2, wl, w, go, cot)
    assert all(np.array_equal(a, b) for a, b in zip(full, again))
    names = ("x", "Y", "w", "g")
    for want in (("x",), ("Y", "w"), ("g",)):
        part, _ = _gpu_dbl(tpc, irr, 2, 2, wl, w, go, cot, want=want)
        for i, nm in enumerate(names):
            assert (part[i] is None) == (nm not in want)
            if nm in want:
                assert np.array_equal(part[i], full[i]), nm
    wl.src, wl.dst, wl.r = wl.src[:0], wl.dst[:0], wl.r[:0]
    cot0 = [cot[0], cot[1][:0], cot[2][:0]]
    empty, _ = _gpu_dbl(tpc, irr, 2, 2, wl, w[:0], go, cot0)
    assert np.all(empty[0] == 0) and np.all(empty[3] == 0)
    assert empty[1].size == 0 and empty[2].size == 0
