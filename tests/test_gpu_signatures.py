"""GPU parity of the 0e+1o signatures at lmax 1 and lmax 3 (node features of
degree <= 1 with harmonics and outputs up to lmax) against the float64
oracle: forward, backward (the one-pass form and the receiver / sender
passes), the edge-vector form and the second-order backward, on a random
graph and on a power-law graph with hubs.  Same bar as the other signatures:
every block within 1e-4 of max|ref| of that block."""
import numpy as np
import pytest

import oracle
from tests._common import dims_of
from tests.test_gpu_parity import T, block_err, in_blocks, out_blocks, say, w_err, y_blocks
from workloads import make_workload

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


def _inputs(U, lmax, graph, n, seed):
    irr = f"{U}x0e+{U}x1o"
    op = oracle.build_plan(irr, lmax, lmax)
    wl = make_workload("mid", dims_of(op), seed=seed, n_nodes=n)
    if graph != "mid":
        gw = make_workload(graph, dims_of(op), seed=seed, n_nodes=n, graph_only=True)
        wl.src, wl.dst, wl.r = gw.src, gw.dst, gw.r
    rng = np.random.default_rng(seed + 3)
    wl.w = (rng.normal(size=(len(wl.src), op.n_paths, U)) / np.sqrt(op.n_paths)).astype(np.float32)
    return irr, op, wl


@pytest.mark.parametrize("U,lmax,graph,n", [(32, 1, "mid", 400), (8, 1, "zipf", 300),
                                            (64, 3, "mid", 300), (16, 3, "zipf", 500),
                                            (128, 3, "lmax3", 120)])
def test_signature_parity(tpc, U, lmax, graph, n):
    say(f"signature 0e+1o lmax {lmax} U={U} graph={graph} n={n}")
    irr, op, wl = _inputs(U, lmax, graph, n, seed=U + lmax)
    plan = tpc.Plan(irr, lmax, lmax)
    g = tpc.graph_build(T(wl.src), T(wl.dst), wl.n_nodes)
    rs = tpc.gather_rows(T(wl.r), g.perm)
    Y = tpc.sph_harm(lmax, rs)
    w = tpc.gather_rows(T(wl.w), g.perm)
    x, go = T(wl.x), T(wl.g)
    out = tpc.forward(plan, g, x, Y, w)
    gx, gY, gw = tpc.backward(plan, g, x, Y, w, go)                         # one pass
    _, gY2, gw2 = tpc.backward(plan, g, x, Y, w, go, want=("Y", "w"))       # receiver pass
    gx2, _, _ = tpc.backward(plan, g, x, Y, w, go, want=("x",))             # sender pass
    out_r = tpc.forward_r(plan, g, x, rs, w)
    gx_r, gr_r, gw_r = tpc.backward_r(plan, g, x, rs, w, go)
    rng = np.random.default_rng(7)
    ggx = rng.normal(size=wl.x.shape).astype(np.float32)
    ggY = rng.normal(size=(wl.n_edges, op.ysh)).astype(np.float32)
    ggw = rng.normal(size=wl.w.shape).astype(np.float32)
    dx, dY, dw, dg = tpc.double_backward(plan, g, x, Y, w, go, T(ggx), tpc.gather_rows(T(ggY), g.perm),
                                         tpc.gather_rows(T(ggw), g.perm))
    torch.cuda.synchronize()
    c = lambda t: t.cpu().numpy()
    p = c(g.perm)[:wl.n_edges]
    Yo = oracle.sh_real(lmax, wl.r)
    ref = oracle.tp_conv_fwd(op, wl.src, wl.dst, wl.n_nodes, wl.x, Yo, wl.w)
    rx, rY, rw = oracle.tp_conv_bwd(op, wl.src, wl.dst, wl.n_nodes, wl.x, Yo, wl.w, wl.g)
    rr = oracle.sh_real_vjp(lmax, wl.r.astype(np.float64), rY)
    for got in (out, out_r):
        assert block_err(c(got), ref, out_blocks(op)) <= TOL
    for got in (gx, gx2, gx_r):
        assert block_err(c(got), rx, in_blocks(op)) <= TOL
    for got in (gY, gY2):
        assert block_err(c(got), rY[p], y_blocks(op)) <= TOL
    for got in (gw, gw2, gw_r):
        assert w_err(c(got), rw[p]) <= TOL
    assert np.max(np.abs(c(gr_r) - rr[p])) <= TOL * np.max(np.abs(rr))
    d = oracle.tp_conv_double_bwd(op, wl.src, wl.dst, wl.n_nodes, wl.x, Yo, wl.w, wl.g, ggx, ggY, ggw)
    assert block_err(c(dx), d[0], in_blocks(op)) <= TOL
    assert block_err(c(dY), d[1][p], y_blocks(op)) <= TOL
    assert w_err(c(dw), d[2][p]) <= TOL
    assert block_err(c(dg), d[3], out_blocks(op)) <= TOL
