"""GPU parity of the sender-grouped edge layout (tp_conv_forward_sg,
tp_conv_backward_sg, tp_conv_graph_sender_positions) against the float64
oracle, through the C ABI.

Edge arrays in this layout hold, at row k, the edge at sender-grouped position
k, i.e. the original edge perm[t_perm[k]].  Bar: every float output within
1e-4 * max|ref| per irrep block (as the receiver-layout tests), e_pos exactly
the inverse of t_perm, and the results bit for bit those of the receiver
layout on the same edges (both sum every receiver's and every sender's edges
in the same order).
"""
import numpy as np
import pytest

import oracle
from tests._common import dims_of
from tests.test_gpu_parity import (T, block_err, dev, in_blocks, out_blocks, plans, say, w_err,
                                   y_blocks)
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


def run_both(tpc, plan, wl, want=("x", "Y", "w")):
    """Receiver layout and sender layout on the same edges; numpy results with
    the sender layout's edge rows and the original edge id of each row."""
    g = tpc.graph_build(T(wl.src), T(wl.dst), wl.n_nodes)
    Y = tpc.sph_harm(plan.lmax_sh, tpc.gather_rows(T(wl.r), g.perm))
    w = tpc.gather_rows(T(wl.w), g.perm)
    x, go = T(wl.x), T(wl.g)
    out = tpc.forward(plan, g, x, Y, w)
    gx, gY, gw = tpc.backward(plan, g, x, Y, w, go)
    e_pos = tpc.graph_sender_positions(g)
    Ys, ws = tpc.gather_rows(Y, g.t_perm), tpc.gather_rows(w, g.t_perm)
    out_s = tpc.forward_sg(plan, g, e_pos, x, Ys, ws)
    gx_s, gY_s, gw_s = tpc.backward_sg(plan, g, x, Ys, ws, go, want=want)
    torch.cuda.synchronize()
    E = wl.n_edges
    n = lambda t: None if t is None else t.cpu().numpy()
    res = dict(out=n(out), gx=n(gx), gY=n(gY), gw=n(gw), out_s=n(out_s), gx_s=n(gx_s), gY_s=n(gY_s),
               gw_s=n(gw_s), e_pos=n(e_pos)[:E], t_perm=n(g.t_perm)[:E], perm=n(g.perm)[:E])
    res["orig"] = res["perm"][res["t_perm"]]      # original edge id of each sender-layout row
    return res


def check_against_oracle(op, wl, res, want=("x", "Y", "w")):
    Y = oracle.sh_real(op.lmax_sh, wl.r)
    ref = oracle.tp_conv_fwd(op, wl.src, wl.dst, wl.n_nodes, wl.x, Y, wl.w)
    assert block_err(res["out_s"], ref, out_blocks(op)) <= TOL
    gx, gY, gw = oracle.tp_conv_bwd(op, wl.src, wl.dst, wl.n_nodes, wl.x, Y, wl.w, wl.g)
    o = res["orig"]
    if "x" in want:
        assert block_err(res["gx_s"], gx, in_blocks(op)) <= TOL
    if "Y" in want:
        assert block_err(res["gY_s"], gY[o], y_blocks(op)) <= TOL
    if "w" in want:
        assert w_err(res["gw_s"], gw[o]) <= TOL


def check_same_as_receiver_layout(res, want=("x", "Y", "w")):
    tp = res["t_perm"]
    assert np.array_equal(res["e_pos"][tp], np.arange(len(tp)))
    assert np.array_equal(res["out_s"], res["out"])
    if "x" in want:
        assert np.array_equal(res["gx_s"], res["gx"])
    if "Y" in want:
        assert np.array_equal(res["gY_s"], res["gY"][tp])
    if "w" in want:
        assert np.array_equal(res["gw_s"], res["gw"][tp])


@pytest.mark.parametrize("name,n_nodes,mul", [
    ("tiny", None, None),
    ("mid", None, None),           # the full 1,536-atom graph
    ("mid", 200, 8),
    ("mid", 1100, 16),             # past the small-graph launch threshold
    ("mid", 200, 64),
    ("stream", 300, None),         # 128 channels
    ("tiny", None, 16),
])
def test_sender_layout_parity(tpc, name, n_nodes, mul):
    say(f"sender layout parity {name} n={n_nodes} mul={mul}")
    plan, op = plans(name, mul)
    wname = "mid" if name == "stream" else name
    wl = make_workload(wname, dims_of(op), n_nodes=n_nodes or (300 if name == "stream" else None))
    res = run_both(tpc, plan, wl)
    check_against_oracle(op, wl, res)
    check_same_as_receiver_layout(res)


def test_sender_layout_hub_graph_and_lmax1(tpc):
    """Power-law receiver degrees (hubs of 100+ edges) with the 32-channel
    signature, and 0e+1o at lmax 1."""
    say("sender layout on a Zipf graph, 1100 nodes")
    plan, op = plans("mid")
    wl = make_workload("mid", dims_of(op), n_nodes=1100, seed=4)
    gz = make_workload("zipf", dims_of(op), n_nodes=1100, seed=4, graph_only=True)
    wl.src, wl.dst, wl.r = gz.src, gz.dst, gz.r
    rng = np.random.default_rng(5)
    wl.w = (rng.normal(size=(len(wl.src), op.n_paths, op.U)) / np.sqrt(op.n_paths)).astype(np.float32)
    assert np.bincount(wl.dst, minlength=wl.n_nodes).max() >= 100
    res = run_both(tpc, plan, wl)
    check_against_oracle(op, wl, res)
    check_same_as_receiver_layout(res)
    say("sender layout 32x0e+32x1o lmax 1")
    import tensor_product_convolution_amd as m
    plan1, op1 = m.Plan("32x0e+32x1o", 1, 1), oracle.build_plan("32x0e+32x1o", 1, 1)
    wl1 = make_workload("mid", dims_of(op1), n_nodes=300, seed=2)
    res1 = run_both(tpc, plan1, wl1)
    check_against_oracle(op1, wl1, res1)
    check_same_as_receiver_layout(res1)


@pytest.mark.parametrize("want", [("x",), ("w",), ("Y",), ("x", "Y"), ("Y", "w")])
def test_sender_layout_output_subsets(tpc, want):
    say(f"sender layout subset {want}")
    plan, op = plans("mid")
    wl = make_workload("mid", dims_of(op), n_nodes=260, seed=3)
    res = run_both(tpc, plan, wl, want=want)
    for k, key in (("x", "gx_s"), ("Y", "gY_s"), ("w", "gw_s")):
        assert (res[key] is None) == (k not in want)
    check_against_oracle(op, wl, res, want)
    check_same_as_receiver_layout(res, want)


def test_sender_layout_empty_hub_and_isolated(tpc):
    say("sender layout empty graph")
    plan, op = plans("mid")
    N = 7
    x = torch.randn(N, op.xdim, device=dev())
    g = tpc.graph_build(T(np.zeros(0, np.int32)), T(np.zeros(0, np.int32)), N)
    e_pos = tpc.graph_sender_positions(g)
    Y = torch.zeros(0, op.ysh, device=dev())
    w = torch.zeros(0, op.n_paths, op.U, device=dev())
    out = torch.full((N, op.outdim), 7.0, device=dev())
    tpc.forward_sg(plan, g, e_pos, x, Y, w, out=out)
    gx = torch.full((N, op.xdim), 7.0, device=dev())
    tpc.backward_sg(plan, g, x, Y, w, torch.randn(N, op.outdim, device=dev()), outs=(gx, None, None))
    torch.cuda.synchronize()
    assert float(out.abs().max()) == 0.0 and float(gx.abs().max()) == 0.0
    say("sender layout hub receiver with isolated nodes")
    rng = np.random.default_rng(3)

    class W:
        pass
    wl = W()
    wl.src = rng.integers(1, 50, 3000).astype(np.int32)
    wl.dst = np.zeros(3000, np.int32)
    wl.r = rng.normal(size=(3000, 3)).astype(np.float32)
    wl.x = rng.normal(size=(50, op.xdim)).astype(np.float32)
    wl.w = (rng.normal(size=(3000, op.n_paths, op.U)) / 4).astype(np.float32)
    wl.g = rng.normal(size=(50, op.outdim)).astype(np.float32)
    wl.n_nodes, wl.n_edges = 50, 3000
    res = run_both(tpc, plan, wl)
    check_against_oracle(op, wl, res)
    check_same_as_receiver_layout(res)
    assert np.all(res["out_s"][1:] == 0)


def test_sender_layout_backward_unsupported_at_lmax3(tpc):
    """The lmax-3 signature has no one-pass backward: the sender layout's
    backward is refused before any launch, its forward still matches."""
    say("sender layout lmax 3")
    plan, op = plans("lmax3", 16)
    wl = make_workload("lmax3", dims_of(op), n_nodes=150, seed=1)
    g = tpc.graph_build(T(wl.src), T(wl.dst), wl.n_nodes)
    Y = tpc.sph_harm(3, tpc.gather_rows(T(wl.r), g.perm))
    w = tpc.gather_rows(T(wl.w), g.perm)
    x = T(wl.x)
    e_pos = tpc.graph_sender_positions(g)
    out = tpc.forward(plan, g, x, Y, w)
    out_s = tpc.forward_sg(plan, g, e_pos, x, tpc.gather_rows(Y, g.t_perm), tpc.gather_rows(w, g.t_perm))
    torch.cuda.synchronize()
    assert torch.equal(out, out_s)
    with pytest.raises(tpc.TPError) as e:
        tpc.backward_sg(plan, g, x, Y, w, T(wl.g))
    assert e.value.status == -3
