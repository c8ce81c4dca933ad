"""GPU parity of the convolution with fully connected per-edge weights (computed
by reassociation into receiver state and a dense contraction) against the
float64 oracle, which forms the per-edge weights and messages by definition.
Every output irrep block within 1e-4 of max|ref| of that block."""
import numpy as np
import pytest

import oracle
from tests._common import dims_of
from tests.test_gpu_parity import T, block_err, out_blocks, say
from workloads import make_fc_inputs, make_workload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 1e-4
H = 8


@pytest.fixture(scope="module")
def tpc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tensor_product_convolution_amd as m
    m.lib()
    return m


def _case(U, graph, n, seed=0):
    irr = f"{U}x0e+{U}x1o+{U}x2e"
    op = oracle.build_plan(irr, 2, 2)
    wl = make_workload("mid", dims_of(op), seed=seed, n_nodes=n)
    if graph != "mid":
        gw = make_workload(graph, dims_of(op), seed=seed, n_nodes=n, graph_only=True)
        wl.src, wl.dst, wl.r = gw.src, gw.dst, gw.r
    R, Th = make_fc_inputs(wl.n_edges, op.n_paths, U, H, seed)
    return irr, op, wl, R, Th


def _gpu(tpc, irr, wl, R, Th):
    plan = tpc.Plan(irr, 2, 2)
    g = tpc.graph_build(T(wl.src), T(wl.dst), wl.n_nodes)
    Y = tpc.sph_harm(2, tpc.gather_rows(T(wl.r), g.perm))
    Rs = tpc.gather_rows(T(R), g.perm)
    out = tpc.forward_fc(plan, g, T(wl.x), Y, Rs, T(Th))
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("U,graph,n", [(16, "mid", 200), (32, "mid", 300), (32, "zipf", 400),
                                       (16, "lmax3", 250), (32, "mid", 1536), (64, "mid", 300),
                                       (64, "zipf", 500)])
def test_fc_forward_parity(tpc, U, graph, n):
    say(f"fc forward U={U} graph={graph} n={n}")
    irr, op, wl, R, Th = _case(U, graph, n)
    got = _gpu(tpc, irr, wl, R, Th)
    ref = oracle.fc_conv_fwd(op, wl.src, wl.dst, wl.n_nodes, wl.x, oracle.sh_real(2, wl.r), R, Th)
    assert block_err(got, ref, out_blocks(op)) <= TOL


def test_fc_isolated_and_empty(tpc):
    say("fc forward isolated nodes, empty graph")
    irr, op, wl, R, Th = _case(32, "mid", 80, seed=3)
    keep = wl.dst >= 10
    wl.src, wl.dst, wl.r = wl.src[keep], wl.dst[keep], wl.r[keep]
    R = R[keep]
    got = _gpu(tpc, irr, wl, R, Th)
    ref = oracle.fc_conv_fwd(op, wl.src, wl.dst, wl.n_nodes, wl.x, oracle.sh_real(2, wl.r), R, Th)
    assert np.all(got[:10] == 0)
    assert block_err(got, ref, out_blocks(op)) <= TOL
    wl.src, wl.dst, wl.r = wl.src[:0], wl.dst[:0], wl.r[:0]
    assert np.all(_gpu(tpc, irr, wl, R[:0], Th) == 0)


def _gpu_bwd(tpc, irr, wl, R, Th, go, want=("x", "Y", "R", "Theta")):
    plan = tpc.Plan(irr, 2, 2)
    g = tpc.graph_build(T(wl.src), T(wl.dst), wl.n_nodes)
    Y = tpc.sph_harm(2, tpc.gather_rows(T(wl.r), g.perm))
    Rs = tpc.gather_rows(T(R), g.perm)
    res = tpc.backward_fc(plan, g, T(wl.x), Y, Rs, T(Th), T(go), want=want)
    torch.cuda.synchronize()
    return [None if r is None else r.cpu().numpy() for r in res], g.perm.cpu().numpy()


def _check_bwd(op, wl, R, Th, go, got, perm):
    gx, gY, gR, gT = got
    rx, rY, rR, rT = oracle.fc_conv_bwd(op, wl.src, wl.dst, wl.n_nodes, wl.x, oracle.sh_real(2, wl.r), R, Th, go)
    xb = [slice(o, o + op.U * (2 * l + 1)) for (_, l, _), o in zip(op.irreps_in, op.in_offsets)]
    yb = [slice(l * l, (l + 1) ** 2) for l in range(3)]
    assert block_err(gx, rx, xb) <= TOL
    assert block_err(gY, rY[perm], yb) <= TOL
    assert block_err(gR, rR[perm], [slice(0, R.shape[1])]) <= TOL
    P, U = op.n_paths, op.U
    assert block_err(gT.reshape(-1, P * U * U), rT.reshape(-1, P * U * U),
                     [slice(p * U * U, (p + 1) * U * U) for p in range(P)]) <= TOL


@pytest.mark.parametrize("U,graph,n", [(16, "mid", 200), (32, "mid", 300), (32, "zipf", 400),
                                       (16, "lmax3", 250), (32, "mid", 1536), (64, "mid", 300),
                                       (64, "lmax3", 200)])
def test_fc_backward_parity(tpc, U, graph, n):
    say(f"fc backward U={U} graph={graph} n={n}")
    irr, op, wl, R, Th = _case(U, graph, n)
    go = np.random.default_rng(7).normal(size=(wl.n_nodes, op.outdim)).astype(np.float32)
    got, perm = _gpu_bwd(tpc, irr, wl, R, Th, go)
    _check_bwd(op, wl, R, Th, go, got, perm)


def test_fc_backward_subsets_isolated_empty(tpc):
    say("fc backward output subsets, isolated nodes, empty graph")
    irr, op, wl, R, Th = _case(32, "mid", 80, seed=3)
    keep = (wl.dst >= 10) & (wl.src >= 5)
    wl.src, wl.dst, wl.r = wl.src[keep], wl.dst[keep], wl.r[keep]
    R = R[keep]
    go = np.random.default_rng(8).normal(size=(wl.n_nodes, op.outdim)).astype(np.float32)
    got, perm = _gpu_bwd(tpc, irr, wl, R, Th, go)
    _check_bwd(op, wl, R, Th, go, got, perm)
    assert np.all(got[0][:5] == 0)
    again, _ = _gpu_bwd(tpc, irr, wl, R, Th, go)
    assert all(np.array_equal(a, b) for a, b in zip(got, again))
    part, _ = _gpu_bwd(tpc, irr, wl, R, Th, go, want=("R",))
    assert part[0] is None and part[1] is None and part[3] is None and np.array_equal(part[2], got[2])
    wl.src, wl.dst, wl.r = wl.src[:0], wl.dst[:0], wl.r[:0]
    empty, _ = _gpu_bwd(tpc, irr, wl, R[:0], Th, go)
    assert np.all(empty[0] == 0) and np.all(empty[3] == 0) and empty[1].size == 0 and empty[2].size == 0


def test_fc_backward_reads_the_saved_state(tpc):
    """With TP_FC_STATE_SAVED the backward reads the state the forward left in
    the shared workspace instead of recomputing it: identical results."""
    say("fc backward with the forward's saved state")
    irr, op, wl, R, Th = _case(32, "mid", 300, seed=5)
    go = T(np.random.default_rng(9).normal(size=(wl.n_nodes, op.outdim)).astype(np.float32))
    plan = tpc.Plan(irr, 2, 2)
    g = tpc.graph_build(T(wl.src), T(wl.dst), wl.n_nodes)
    Y = tpc.sph_harm(2, tpc.gather_rows(T(wl.r), g.perm))
    Rs, x, Tt = tpc.gather_rows(T(R), g.perm), T(wl.x), T(Th)
    ws = torch.empty(tpc.fc_backward_workspace(plan, wl.n_nodes, H), dtype=torch.uint8, device=x.device)
    ref = tpc.backward_fc(plan, g, x, Y, Rs, Tt, go)
    tpc.forward_fc(plan, g, x, Y, Rs, Tt, ws=ws)
    got = tpc.backward_fc(plan, g, x, Y, Rs, Tt, go, ws=ws, state_saved=True)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(got, ref))
    with pytest.raises(ValueError):
        tpc.backward_fc(plan, g, x, Y, Rs, Tt, go, state_saved=True)


def _gpu_dbl(tpc, irr, wl, R, Th, go, cot, want=("x", "Y", "R", "Theta", "g")):
    """second-order backward on the GPU; edge cotangents in original order"""
    plan = tpc.Plan(irr, 2, 2)
    g = tpc.graph_build(T(wl.src), T(wl.dst), wl.n_nodes)
    Y = tpc.sph_harm(2, tpc.gather_rows(T(wl.r), g.perm))
    Rs = tpc.gather_rows(T(R), g.perm)
    ggx, ggY, ggR, ggT = cot
    gath = lambda a: None if a is None else tpc.gather_rows(T(a), g.perm)
    res = tpc.double_backward_fc(plan, g, T(wl.x), Y, Rs, T(Th), T(go),
                                 gg_x=None if ggx is None else T(ggx), gg_Y=gath(ggY), gg_R=gath(ggR),
                                 gg_Theta=None if ggT is None else T(ggT), want=want)
    torch.cuda.synchronize()
    return [None if r is None else r.cpu().numpy() for r in res], g.perm.cpu().numpy()


def _check_dbl(op, wl, R, Th, go, cot, got, perm):
    ref = oracle.fc_conv_double_bwd(op, wl.src, wl.dst, wl.n_nodes, wl.x, oracle.sh_real(2, wl.r), R, Th, go,
                                    *cot)
    dx, dY, dR, dT, dg = got
    xb = [slice(o, o + op.U * (2 * l + 1)) for (_, l, _), o in zip(op.irreps_in, op.in_offsets)]
    yb = [slice(l * l, (l + 1) ** 2) for l in range(3)]
    P, U = op.n_paths, op.U
    if dx is not None:
        assert block_err(dx, ref[0], xb) <= TOL, "d_x"
    if dY is not None:
        assert block_err(dY, ref[1][perm], yb) <= TOL, "d_Y"
    if dR is not None:
        assert block_err(dR, ref[2][perm], [slice(0, R.shape[1])]) <= TOL, "d_R"
    if dT is not None:
        assert block_err(dT.reshape(-1, P * U * U), ref[3].reshape(-1, P * U * U),
                         [slice(p * U * U, (p + 1) * U * U) for p in range(P)]) <= TOL, "d_Theta"
    if dg is not None:
        assert block_err(dg, ref[4], out_blocks(op)) <= TOL, "d_grad_out"


def _fc_cotangents(op, wl, R, Th, seed):
    rng = np.random.default_rng(seed)
    f = lambda shape: rng.normal(size=shape).astype(np.float32)
    return [f(wl.x.shape), f((wl.n_edges, op.ysh)), f(R.shape), (f(Th.shape) / op.U).astype(np.float32)]


@pytest.mark.parametrize("U,graph,n", [(16, "mid", 200), (32, "zipf", 400), (32, "lmax3", 600),
                                       (64, "mid", 200)])
def test_fc_double_backward_parity(tpc, U, graph, n):
    say(f"fc double backward U={U} graph={graph} n={n}")
    irr, op, wl, R, Th = _case(U, graph, n)
    go = np.random.default_rng(9).normal(size=(wl.n_nodes, op.outdim)).astype(np.float32)
    cot = _fc_cotangents(op, wl, R, Th, U + n)
    got, perm = _gpu_dbl(tpc, irr, wl, R, Th, go, cot)
    _check_dbl(op, wl, R, Th, go, cot, got, perm)


def test_fc_double_backward_missing_cotangents_subsets_degenerate(tpc):
    """Each cotangent alone, none (zeros), output subsets, determinism, isolated
    nodes and the empty graph."""
    say("fc double backward: cotangent and output subsets, degenerate graphs")
    irr, op, wl, R, Th = _case(16, "mid", 90, seed=5)
    keep = (wl.dst >= 10) & (wl.src >= 5)
    wl.src, wl.dst, wl.r = wl.src[keep], wl.dst[keep], wl.r[keep]
    R = R[keep]
    go = np.random.default_rng(10).normal(size=(wl.n_nodes, op.outdim)).astype(np.float32)
    cot = _fc_cotangents(op, wl, R, Th, 41)
    for k in range(4):
        one = [c if i == k else None for i, c in enumerate(cot)]
        got, perm = _gpu_dbl(tpc, irr, wl, R, Th, go, one)
        _check_dbl(op, wl, R, Th, go, one, got, perm)
    none, _ = _gpu_dbl(tpc, irr, wl, R, Th, go, [None] * 4)
    assert all(np.all(a == 0) for a in none)
    full, perm = _gpu_dbl(tpc, irr, wl, R, Th, go, cot)
    _check_dbl(op, wl, R, Th, go, cot, full, perm)
    assert np.all(full[0][:5] == 0) and np.all(full[4][:10] == 0)
    again, _ = _gpu_dbl(tpc, irr, wl, R, Th, go, cot)
    assert all(np.array_equal(a, b) for a, b in zip(full, again))
    names = ("x", "Y", "R", "Theta", "g")
    for want in (("x",), ("Y", "R"), ("Theta",), ("g",)):
        part, _ = _gpu_dbl(tpc, irr, wl, R, Th, go, cot, want=want)
        for i, nm in enumerate(names):
            assert (part[i] is None) == (nm not in want)
            if nm in want:
                assert np.array_equal(part[i], full[i]), nm
    wl.src, wl.dst, wl.r = wl.src[:0], wl.dst[:0], wl.r[:0]
    cot0 = [cot[0], cot[1][:0], cot[2][:0], cot[3]]
    empty, _ = _gpu_dbl(tpc, irr, wl, R[:0], Th, go, cot0)
    assert np.all(empty[0] == 0) and np.all(empty[3] == 0) and np.all(empty[4] == 0)
    assert empty[1].size == 0 and empty[2].size == 0
