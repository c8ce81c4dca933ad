"""GPU parity of the second-order backward (the gradients of a loss on the first
backward's outputs) against the float64 oracle, every output block within 1e-4 of
max|ref| of that block, on the direct-weight workloads at test sizes, with hub
degrees, with missing cotangents, and on a graph with isolated nodes."""
import numpy as np
import pytest

import oracle
from tests._common import dims_of
from tests.test_gpu_parity import T, block_err, in_blocks, out_blocks, plans, say, w_err, y_blocks
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


def _run(tpc, plan, wl, cot, which=("x", "Y", "w")):
    g = tpc.graph_build(T(wl.src), T(wl.dst), wl.n_nodes)
    Y = tpc.sph_harm(plan.lmax_sh, tpc.gather_rows(T(wl.r), g.perm))
    w = tpc.gather_rows(T(wl.w), g.perm)
    ggx = T(cot["x"]) if "x" in which else None
    ggY = tpc.gather_rows(T(cot["Y"]), g.perm) if "Y" in which else None
    ggw = tpc.gather_rows(T(cot["w"]), g.perm) if "w" in which else None
    dx, dY, dw, dg = tpc.double_backward(plan, g, T(wl.x), Y, w, T(wl.g), ggx, ggY, ggw)
    torch.cuda.synchronize()
    p = g.perm.cpu().numpy()[:wl.n_edges]
    return p, dx.cpu().numpy(), dY.cpu().numpy(), dw.cpu().numpy(), dg.cpu().numpy()


def _cotangents(op, wl, seed):
    rng = np.random.default_rng(seed)
    f = lambda *s: rng.normal(size=s).astype(np.float32)
    return {"x": f(wl.n_nodes, op.xdim), "Y": f(wl.n_edges, op.ysh),
            "w": f(wl.n_edges, op.n_paths, op.U)}


def _check(op, wl, cot, res, which):
    p, dx, dY, dw, dg = res
    Yo = oracle.sh_real(op.lmax_sh, wl.r)
    ref = oracle.tp_conv_double_bwd(op, wl.src, wl.dst, wl.n_nodes, wl.x, Yo, wl.w, wl.g,
                                    cot["x"] if "x" in which else None,
                                    cot["Y"] if "Y" in which else None,
                                    cot["w"] if "w" in which else None)
    rx, rY, rw, rg = ref
    if np.any(rx):
        assert block_err(dx, rx, in_blocks(op)) <= TOL
    else:
        assert np.all(dx == 0)
    assert block_err(dY, rY[p], y_blocks(op)) <= TOL
    assert w_err(dw, rw[p]) <= TOL
    assert block_err(dg, rg, out_blocks(op)) <= TOL


@pytest.mark.parametrize("name,n_nodes,mul", [("tiny", None, None), ("mid", 200, None),
                                              ("mid", 1536, None),
                                              ("lmax3", 120, None), ("zipf", 300, None),
                                              ("stream", 100, None)])
def test_double_backward_parity(tpc, name, n_nodes, mul):
    say(f"double backward {name} n={n_nodes}")
    plan, op = plans(name, mul)
    wname = "mid" if name == "stream" else name
    wl = make_workload(wname, dims_of(op), n_nodes=n_nodes or (100 if name == "stream" else None))
    if wl.g is None:
        wl.g = np.random.default_rng(5).normal(size=(wl.n_nodes, op.outdim)).astype(np.float32)
    cot = _cotangents(op, wl, 7)
    _check(op, wl, cot, _run(tpc, plan, wl, cot), ("x", "Y", "w"))


@pytest.mark.parametrize("which", [("x",), ("Y",), ("w",), ("Y", "w")])
def test_double_backward_missing_cotangents(tpc, which):
    say(f"double backward cotangents {which}")
    plan, op = plans("mid")
    wl = make_workload("mid", dims_of(op), n_nodes=150)
    cot = _cotangents(op, wl, 8)
    _check(op, wl, cot, _run(tpc, plan, wl, cot, which), which)


@pytest.mark.parametrize("want", [("g",), ("Y", "w"), ("x", "w"), ("Y",)])
def test_double_backward_output_subsets(tpc, want):
    """Requesting only some outputs gives those outputs bit for bit as the full
    call does (the receiver pass branches on which of dg, dY and dw are asked
    for); the full call is the one checked against the oracle above."""
    say(f"double backward outputs {want}")
    plan, op = plans("mid")
    wl = make_workload("mid", dims_of(op), n_nodes=150)
    cot = _cotangents(op, wl, 9)
    g = tpc.graph_build(T(wl.src), T(wl.dst), wl.n_nodes)
    Y = tpc.sph_harm(plan.lmax_sh, tpc.gather_rows(T(wl.r), g.perm))
    w = tpc.gather_rows(T(wl.w), g.perm)
    args = (plan, g, T(wl.x), Y, w, T(wl.g), T(cot["x"]), tpc.gather_rows(T(cot["Y"]), g.perm),
            tpc.gather_rows(T(cot["w"]), g.perm))
    full = tpc.double_backward(*args)
    part = tpc.double_backward(*args, want=want)
    torch.cuda.synchronize()
    for k, a, b in zip("xYwg", full, part):
        if k in want:
            assert torch.equal(a, b), k
        else:
            assert b is None


def test_double_backward_hub_isolated_and_empty(tpc):
    """One receiver with 3,000 edges (its walk split over the waves of its
    workgroup), 49 receivers and one sender without edges, against the oracle;
    then a graph with no edges, whose node outputs are zeros."""
    say("double backward hub receiver, isolated nodes")
    plan, op = plans("mid")
    rng = np.random.default_rng(11)

    class W:
        pass
    wl = W()
    wl.n_nodes, wl.n_edges = 50, 3000
    wl.src = rng.integers(1, 50, 3000).astype(np.int32)
    wl.dst = np.zeros(3000, np.int32)
    wl.r = rng.normal(size=(3000, 3)).astype(np.float32)
    wl.x = rng.normal(size=(50, op.xdim)).astype(np.float32)
    wl.w = (rng.normal(size=(3000, op.n_paths, op.U)) / 4).astype(np.float32)
    wl.g = rng.normal(size=(50, op.outdim)).astype(np.float32)
    cot = _cotangents(op, wl, 12)
    res = _run(tpc, plan, wl, cot)
    _check(op, wl, cot, res, ("x", "Y", "w"))
    _, dx, _, _, dg = res
    assert np.all(dg[1:] == 0) and np.all(dx[0] == 0)

    say("double backward empty graph")
    N = 7
    g = tpc.graph_build(T(np.zeros(0, np.int32)), T(np.zeros(0, np.int32)), N)
    Y = torch.zeros(0, op.ysh, device="cuda")
    w = torch.zeros(0, op.n_paths, op.U, device="cuda")
    x = torch.randn(N, op.xdim, device="cuda")
    gout = torch.randn(N, op.outdim, device="cuda")
    dx, dY, dw, dg = tpc.double_backward(plan, g, x, Y, w, gout, torch.randn_like(x), Y, w)
    torch.cuda.synchronize()
    assert float(dx.abs().max()) == 0.0 and float(dg.abs().max()) == 0.0
    assert dY.shape == (0, op.ysh) and dw.shape == (0, op.n_paths, op.U)
