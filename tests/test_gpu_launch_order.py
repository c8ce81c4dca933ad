"""GPU: launch orders (tp_conv_graph_launch_order) and the convolution with
them, through the C ABI.

Bar: order / t_order bit for bit those of the oracle (nodes by descending
degree, ties by node id) on every workload's graph and on edge cases; the
forward, the backward (one-pass, two-pass, edge-vector and sender-grouped
forms) bit for bit the same with and without a launch order, and within 1e-4
* max|ref| per irrep block of the float64 oracle; the second-order backward
bit for bit the same with and without a launch order.
"""
import numpy as np
import pytest

import oracle
from tests._common import dims_of
from tests.test_gpu_parity import (T, block_err, in_blocks, out_blocks, plans, say, w_err, y_blocks)
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


def check_orders(tpc, src, dst, n):
    g = tpc.graph_launch_order(tpc.graph_build(T(np.asarray(src, np.int32)), T(np.asarray(dst, np.int32)), n))
    torch.cuda.synchronize()
    ref = oracle.csr_build(src, dst, n)
    assert np.array_equal(g.order.cpu().numpy(), oracle.launch_order(ref["row_ptr"]))
    assert np.array_equal(g.t_order.cpu().numpy(), oracle.launch_order(ref["t_row_ptr"]))
    return g


@pytest.mark.parametrize("name", ["tiny", "mid", "lmax3", "zipf", "stream"])
def test_launch_order_bit_exact_full_size(tpc, name):
    say(f"launch order {name}")
    wl = make_workload(name, dict(xdim=0, n_paths=0, U=0, outdim=0, n_out_irreps=0), graph_only=True)
    check_orders(tpc, wl.src, wl.dst, wl.n_nodes)


def test_launch_order_edge_cases(tpc):
    rng = np.random.default_rng(0)
    say("launch order edge cases")
    check_orders(tpc, np.zeros(0, np.int32), np.zeros(0, np.int32), 5)            # no edges: node order
    check_orders(tpc, [0, 0, 0], [0, 0, 0], 1)                                    # one node
    check_orders(tpc, rng.integers(0, 50, 7000), np.zeros(7000, np.int64), 50)    # one hub
    check_orders(tpc, rng.integers(0, 300000, 5000), rng.integers(0, 300000, 5000), 300000)  # 3 passes
    # one grouping only
    g = tpc.graph_build(T(np.array([1, 2, 2], np.int32)), T(np.array([0, 0, 1], np.int32)), 3)
    tpc.graph_launch_order(g, senders=False)
    torch.cuda.synchronize()
    assert g.t_order is None and g.order.cpu().tolist() == [0, 1, 2]
    tpc.graph_launch_order(g, receivers=False)
    torch.cuda.synchronize()
    assert g.order is None and g.t_order.cpu().tolist() == [2, 1, 0]


def run(tpc, plan, wl, ordered, forms=("y", "r", "sg")):
    g = tpc.graph_build(T(wl.src), T(wl.dst), wl.n_nodes)
    if ordered:
        tpc.graph_launch_order(g)
    r = tpc.gather_rows(T(wl.r), g.perm)
    Y = tpc.sph_harm(plan.lmax_sh, r)
    w = tpc.gather_rows(T(wl.w), g.perm)
    x, go = T(wl.x), T(wl.g)
    res = {"out": tpc.forward(plan, g, x, Y, w)}
    res["gx"], res["gY"], res["gw"] = tpc.backward(plan, g, x, Y, w, go)
    # each pass alone (the two-pass form's receiver and sender passes)
    res["gx_only"] = tpc.backward(plan, g, x, Y, w, go, want=("x",))[0]
    res["gw_only"] = tpc.backward(plan, g, x, Y, w, go, want=("w",))[2]
    # second order, the first-order outputs as cotangents
    res["dx"], res["dY"], res["dw"], res["dg"] = tpc.double_backward(plan, g, x, Y, w, go, res["gx"],
                                                                     res["gY"], res["gw"])
    if "r" in forms:
        res["out_r"] = tpc.forward_r(plan, g, x, r, w)
        res["gx_r"], res["gr_r"], res["gw_r"] = tpc.backward_r(plan, g, x, r, w, go)
    if "sg" in forms:
        e_pos = tpc.graph_sender_positions(g)
        Ys, ws = tpc.gather_rows(Y, g.t_perm), tpc.gather_rows(w, g.t_perm)
        res["out_sg"] = tpc.forward_sg(plan, g, e_pos, x, Ys, ws)
        res["gx_sg"], res["gY_sg"], res["gw_sg"] = tpc.backward_sg(plan, g, x, Ys, ws, go)
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in res.items()}
    out["perm"] = g.perm.cpu().numpy()[:wl.n_edges]
    return out


@pytest.mark.parametrize("name,n_nodes,mul,zipf_graph", [
    ("mid", None, None, False),        # the full 1,536-atom graph
    ("mid", 1100, None, True),         # hubs past the small-graph threshold
    ("mid", 300, 128, False),
    ("tiny", None, None, False),       # small-graph launch shape
    ("lmax3", 600, 16, True),          # two-pass backward on a power-law graph
])
def test_conv_with_launch_order(tpc, name, n_nodes, mul, zipf_graph):
    say(f"conv with launch order {name} n={n_nodes} mul={mul} zipf={zipf_graph}")
    plan, op = plans(name, mul)
    wl = make_workload(name, dims_of(op), n_nodes=n_nodes, seed=4)
    if zipf_graph:
        gz = make_workload("zipf", dims_of(op), n_nodes=wl.n_nodes, seed=4, graph_only=True)
        wl.src, wl.dst, wl.r = gz.src, gz.dst, gz.r
        rng = np.random.default_rng(5)
        wl.w = (rng.normal(size=(len(wl.src), op.n_paths, op.U)) / np.sqrt(op.n_paths)).astype(np.float32)
    forms = ("y", "r") if op.lmax_sh == 3 else ("y", "r", "sg")
    a = run(tpc, plan, wl, False, forms)
    b = run(tpc, plan, wl, True, forms)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    Y = oracle.sh_real(op.lmax_sh, wl.r)
    ref = oracle.tp_conv_fwd(op, wl.src, wl.dst, wl.n_nodes, wl.x, Y, wl.w)
    assert block_err(b["out"], ref, out_blocks(op)) <= TOL
    gx, gY, gw = oracle.tp_conv_bwd(op, wl.src, wl.dst, wl.n_nodes, wl.x, Y, wl.w, wl.g)
    p = b["perm"]
    assert block_err(b["gx"], gx, in_blocks(op)) <= TOL
    assert block_err(b["gY"], gY[p], y_blocks(op)) <= TOL
    assert w_err(b["gw"], gw[p]) <= TOL


@pytest.mark.parametrize("U,lsh,graph,n", [(16, 3, "zipf", 400), (16, 3, "lmax3", 1100),
                                           (128, 2, "lmax3", 150)])
def test_radial_layer_with_launch_order(tpc, U, lsh, graph, n):
    """The radial-weight layer with a launch order: per-node and per-edge
    outputs bit for bit those in node order (each node is still formed by one
    lane group or wave), the parameter gradients, whose per-wave partial sums
    now collect other nodes, within the bar of the oracle."""
    from tests.test_gpu_radial import _check_params, _vec_err
    say(f"radial layer with launch order U={U} lmax={lsh} graph={graph} n={n}")
    irr = "+".join(f"{U}x{l}{'e' if l % 2 == 0 else 'o'}" for l in range(lsh + 1))
    op = oracle.build_plan(irr, lsh, lsh)
    wl = make_workload("stream", dims_of(op), seed=U + n, n_nodes=n)
    gw = make_workload(graph, dims_of(op), seed=U + n, n_nodes=n, graph_only=True)
    wl.src, wl.dst, wl.r = gw.src, gw.dst, gw.r
    plan = tpc.Plan(irr, lsh, lsh, radial=(8, 64, 5.0), uvw=True)
    res = []
    for ordered in (False, True):
        g = tpc.graph_build(T(wl.src), T(wl.dst), wl.n_nodes)
        if ordered:
            tpc.graph_launch_order(g)
        Y = tpc.sph_harm(lsh, tpc.gather_rows(T(wl.r), g.perm))
        rl = tpc.gather_rows(T(wl.r_len), g.perm)
        x, W1, W2, Wm, go = T(wl.x), T(wl.W1), T(wl.W2), T(wl.Wmix), T(wl.g)
        out, pre = tpc.forward_radial(plan, g, x, Y, rl, W1, W2, Wm)
        b = tpc.backward_radial(plan, g, x, Y, rl, W1, W2, go, Wmix=Wm, out_pre=pre,
                                want=("x", "Y", "W1", "W2", "Wmix", "rlen"))
        torch.cuda.synchronize()
        res.append([t.cpu().numpy() for t in (out, pre) + tuple(b)] + [g.perm.cpu().numpy()[:wl.n_edges]])
    a, o = res
    for k, name in enumerate(("out", "out_pre", "grad_x", "grad_Y")):
        assert np.array_equal(a[k], o[k]), name
    assert np.array_equal(a[7], o[7])                                   # grad_rlen
    Yo = oracle.sh_real(lsh, wl.r)
    rb = oracle.tp_conv_radial_bwd(op, wl.src, wl.dst, wl.n_nodes, wl.x, Yo, wl.r_len, wl.W1, wl.W2, wl.Wmix,
                                   wl.g, 8, 5.0, with_grad_rlen=True)
    p = o[8]
    assert block_err(o[2], rb[0], in_blocks(op)) <= TOL
    assert block_err(o[3], rb[1][p], y_blocks(op)) <= TOL
    assert _vec_err(o[7], rb[5][p]) <= TOL
    _check_params(op, dict(gW1=o[4], gW2=o[5], gWm=o[6]), rb, U)


@pytest.mark.parametrize("U,lsh,graph,n", [(16, 2, "zipf", 400), (16, 3, "lmax3", 300)])
def test_radial_double_backward_with_launch_order(tpc, U, lsh, graph, n):
    """Second-order backward of the radial layer with a launch order: per-node
    and per-edge outputs bit for bit those in node order, all outputs within
    the bar of the oracle."""
    from tests.test_gpu_radial_double import _check, _cotangents, _ref
    say(f"radial double backward with launch order U={U} lmax={lsh} graph={graph} n={n}")
    irr = "+".join(f"{U}x{l}{'e' if l % 2 == 0 else 'o'}" for l in range(lsh + 1))
    op = oracle.build_plan(irr, lsh, lsh)
    wl = make_workload("stream", dims_of(op), seed=U + n, n_nodes=n)
    gw = make_workload(graph, dims_of(op), seed=U + n, n_nodes=n, graph_only=True)
    wl.src, wl.dst, wl.r = gw.src, gw.dst, gw.r
    plan = tpc.Plan(irr, lsh, lsh, radial=(8, 64, 5.0), uvw=True)
    ggx, ggY, ggr = _cotangents(op, wl.n_nodes, wl.n_edges, U + n)
    names = ("dx", "dY", "drl", "dW1", "dW2", "dWm", "dg")
    res = []
    for ordered in (False, True):
        g = tpc.graph_build(T(wl.src), T(wl.dst), wl.n_nodes)
        if ordered:
            tpc.graph_launch_order(g)
        Y = tpc.sph_harm(lsh, tpc.gather_rows(T(wl.r), g.perm))
        rl = tpc.gather_rows(T(wl.r_len), g.perm)
        out = tpc.double_backward_radial(plan, g, T(wl.x), Y, rl, T(wl.W1), T(wl.W2), T(wl.g), Wmix=T(wl.Wmix),
                                         gg_x=T(ggx), gg_Y=tpc.gather_rows(T(ggY), g.perm),
                                         gg_rlen=tpc.gather_rows(T(ggr), g.perm))
        torch.cuda.synchronize()
        r = {k: v.cpu().numpy() for k, v in zip(names, out)}
        r["perm"] = g.perm.cpu().numpy()[:wl.n_edges]
        res.append(r)
    a, o = res
    for k in ("dx", "dY", "drl", "dg"):
        assert np.array_equal(a[k], o[k]), k
    _check(op, o, _ref(op, wl, True, wl.g, ggx, ggY, ggr, lmax=lsh), U, o["perm"])


def test_fc_and_gaunt_with_launch_order(tpc):
    """The fully connected family and the Gaunt product on a power-law graph
    with a launch order: forward and backward bit for bit those in node order,
    and within the bar of the oracle."""
    from tests.test_gpu_fc import _case as fc_case, _check_bwd as fc_check
    from tests.test_gpu_gaunt import _bwd_blocks, _blocks, _case as gaunt_case
    say("fc with launch order, U=32 zipf 400")
    irr, op, wl, R, Th = fc_case(32, "zipf", 400)
    go = np.random.default_rng(7).normal(size=(wl.n_nodes, op.outdim)).astype(np.float32)
    res = []
    for ordered in (False, True):
        plan = tpc.Plan(irr, 2, 2)
        g = tpc.graph_build(T(wl.src), T(wl.dst), wl.n_nodes)
        if ordered:
            tpc.graph_launch_order(g)
        Y = tpc.sph_harm(2, tpc.gather_rows(T(wl.r), g.perm))
        Rs = tpc.gather_rows(T(R), g.perm)
        out = tpc.forward_fc(plan, g, T(wl.x), Y, Rs, T(Th))
        b = tpc.backward_fc(plan, g, T(wl.x), Y, Rs, T(Th), T(go))
        torch.cuda.synchronize()
        res.append([out.cpu().numpy()] + [t.cpu().numpy() for t in b] + [g.perm.cpu().numpy()])
    for k in range(5):
        assert np.array_equal(res[0][k], res[1][k]), k
    ref = oracle.fc_conv_fwd(op, wl.src, wl.dst, wl.n_nodes, wl.x, oracle.sh_real(2, wl.r), R, Th)
    assert block_err(res[1][0], ref, out_blocks(op)) <= TOL
    fc_check(op, wl, R, Th, go, res[1][1:5], res[1][5])

    say("gaunt with launch order, U=32 zipf 400")
    irr = "32x0e+32x1o+32x2e"
    gp, wl, w = gaunt_case(irr, 2, 2, "zipf", 400)
    go = np.random.default_rng(11).normal(size=(wl.n_nodes, gp.outdim)).astype(np.float32)
    res = []
    for ordered in (False, True):
        plan = tpc.Plan(irr, 2, 2, mode=tpc.TP_MODE_GAUNT)
        g = tpc.graph_build(T(wl.src), T(wl.dst), wl.n_nodes)
        if ordered:
            tpc.graph_launch_order(g)
        Y = tpc.sph_harm(2, tpc.gather_rows(T(wl.r), g.perm))
        ws = tpc.gather_rows(T(w.reshape(w.shape[0], w.shape[1] * w.shape[2])), g.perm)
        out = tpc.forward_gaunt(plan, g, T(wl.x), Y, ws)
        b = tpc.backward_gaunt(plan, g, T(wl.x), Y, ws, T(go))
        torch.cuda.synchronize()
        res.append([out.cpu().numpy()] + [t.cpu().numpy() for t in b] + [g.perm.cpu().numpy()])
    for k in range(4):
        assert np.array_equal(res[0][k], res[1][k]), k
    o = res[1]
    ref = oracle.gaunt_conv_fwd(gp, wl.src, wl.dst, wl.n_nodes, wl.x, oracle.sh_real(2, wl.r), w)
    assert block_err(o[0], ref, _blocks(gp)) <= TOL
    rx, rY, rw = oracle.gaunt_conv_bwd(gp, wl.src, wl.dst, wl.n_nodes, wl.x, oracle.sh_real(2, wl.r), w, go)
    xb, yb, wb = _bwd_blocks(gp, wl.n_edges)
    perm = o[4][:wl.n_edges]
    assert block_err(o[1], rx, xb) <= TOL
    assert block_err(o[2], rY[perm], yb) <= TOL
    assert block_err(o[3], rw.reshape(len(rw), -1)[perm], wb) <= TOL
