"""The forward + backward step captured once in a HIP graph (torch's stream
capture around the C-ABI calls) and replayed: every replay, with eager work of
the program and synchronisations between replays, gives exactly the eager
results.  The step's calls launch kernels only (no memset, no allocation, no
host synchronisation), so they can be captured."""
import numpy as np
import pytest

from tests.test_gpu_parity import T, plans, say
from workloads import make_workload
from tests._common import dims_of

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tpc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tensor_product_convolution_amd as m
    m.lib()
    return m


@pytest.mark.parametrize("name,n_nodes", [("mid", 1100), ("tiny", None), ("lmax3", 200)])
def test_step_replays_from_a_hip_graph(tpc, name, n_nodes):
    say(f"graph replay {name} n={n_nodes}")
    plan, op = plans(name)
    wl = make_workload(name, dims_of(op), n_nodes=n_nodes)
    g = tpc.graph_build(T(wl.src), T(wl.dst), wl.n_nodes)
    Y = tpc.sph_harm(plan.lmax_sh, tpc.gather_rows(T(wl.r), g.perm))
    w = tpc.gather_rows(T(wl.w), g.perm)
    x, go = T(wl.x), T(wl.g)
    ref = [tpc.forward(plan, g, x, Y, w), *tpc.backward(plan, g, x, Y, w, go)]
    out, gx, gY, gw = [torch.empty_like(r) for r in ref]

    def step():
        tpc.forward(plan, g, x, Y, w, out=out)
        tpc.backward(plan, g, x, Y, w, go, outs=(gx, gY, gw))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                   # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    hg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(hg):
        step()
    x2 = x * 0.5
    for rep in range(4):
        for t in (out, gx, gY, gw):
            t.fill_(float("nan"))                # eager work between replays
        tpc.forward(plan, g, x2, Y, w)           # an eager call of the library itself
        torch.cuda.synchronize()
        hg.replay()
        torch.cuda.synchronize()
        for got, want in zip((out, gx, gY, gw), ref):
            assert torch.equal(got, want), f"replay {rep}"


@pytest.mark.parametrize("irreps,lmax,n", [("16x0e+16x1o+16x2e", 2, 300), ("16x0e+16x1o+16x2e+16x3o", 3, 200)])
def test_radial_step_replays_from_a_hip_graph(tpc, irreps, lmax, n):
    """The radial layer's step (forward with the channel mix, then all first-order
    gradients) captured once and replayed: bitwise the eager results, with
    eager work between replays.  Outputs and workspace are allocated before
    the capture."""
    import oracle
    say(f"graph replay radial lmax {lmax} n={n}")
    plan = tpc.Plan(irreps, lmax, lmax, radial=(8, 64, 5.0), uvw=True)
    op = oracle.build_plan(irreps, lmax, lmax)
    wl = make_workload("stream", dims_of(op), seed=9, n_nodes=n)
    g = tpc.graph_build(T(wl.src), T(wl.dst), wl.n_nodes)
    Y = tpc.sph_harm(lmax, tpc.gather_rows(T(wl.r), g.perm))
    rl = tpc.gather_rows(T(wl.r_len), g.perm)
    x, W1, W2, Wm, go = T(wl.x), T(wl.W1), T(wl.W2), T(wl.Wmix), T(wl.g)
    want = ("x", "Y", "W1", "W2", "Wmix", "rlen")
    ref_out, ref_pre = tpc.forward_radial(plan, g, x, Y, rl, W1, W2, Wm)
    ref = tpc.backward_radial(plan, g, x, Y, rl, W1, W2, go, Wmix=Wm, out_pre=ref_pre, want=want)
    out, pre = torch.empty_like(ref_out), torch.empty_like(ref_pre)
    outs = {k: torch.empty_like(v) for k, v in zip(want, ref)}
    ws = torch.empty(tpc.radial_workspace(plan, wl.n_nodes, True), dtype=torch.uint8, device=x.device)

    def step():
        tpc.forward_radial(plan, g, x, Y, rl, W1, W2, Wm, out=out, out_pre=pre)
        tpc.backward_radial(plan, g, x, Y, rl, W1, W2, go, Wmix=Wm, out_pre=pre, want=want, outs=outs, ws=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    hg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(hg):
        step()
    for rep in range(4):
        for t in (out, pre, *outs.values()):
            t.fill_(float("nan"))
        tpc.forward_radial(plan, g, x * 0.5, Y, rl, W1, W2, Wm)     # an eager call in between
        torch.cuda.synchronize()
        hg.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(pre, ref_pre), f"replay {rep}"
        for k, r in zip(want, ref):
            assert torch.equal(outs[k], r), f"replay {rep}: grad {k}"
