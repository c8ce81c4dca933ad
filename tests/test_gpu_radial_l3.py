"""GPU parity of the streaming radial-weight layer at lmax 3 (signature
0e+1o+2e+3o with harmonics and outputs up to l = 3, 34 paths) against the
float64 oracle: forward with and without the channel mix, the backward
(grad_x, grad_Y, grad_r_len, grad_W1, grad_W2 per path, grad_Wmix, forces) and
the edge-vector forms, on graphs with uniform degrees 5..30, a hub-heavy
power law, and a 4,200-atom graph that fills the persistent grids of the
receiver pass (512 workgroups of eight waves) and of the grad_W2 pass; and
the second-order backward (cotangents on grad_x, grad_Y and grad_r_len), incl.
a 1,100-atom graph that fills its receiver pass's grid.  Same bar as the
other signatures: every block within 1e-4 of max|ref| of that block."""
import numpy as np
import pytest

import oracle
from tests._common import dims_of
from tests.test_gpu_parity import T, block_err, in_blocks, out_blocks, say, y_blocks
from tests.test_gpu_radial import _check_params, _vec_err
from workloads import make_workload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 1e-4
RC = 5.0


@pytest.fixture(scope="module")
def tpc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tensor_product_convolution_amd as m
    m.lib()
    return m


def _irreps(U):
    return f"{U}x0e+{U}x1o+{U}x2e+{U}x3o"


def _inputs(U, graph, n, seed):
    op = oracle.build_plan(_irreps(U), 3, 3)
    dims = dims_of(op)
    wl = make_workload("stream", dims, seed=seed, n_nodes=n)       # radial parameters
    gw = make_workload(graph, dims, seed=seed, n_nodes=n, graph_only=True)
    wl.src, wl.dst, wl.r = gw.src, gw.dst, gw.r
    return op, wl


def _forces_ref(r, gY, grl):
    r = r.astype(np.float64)
    return oracle.sh_real_vjp(3, r, gY) + grl[:, None] * r / np.linalg.norm(r, axis=1)[:, None]


@pytest.mark.parametrize("U,graph,n,mix", [(16, "zipf", 400, False), (32, "stream", 200, True),
                                           (64, "lmax3", 150, True), (16, "lmax3", 4200, True)])
def test_radial_l3_parity(tpc, U, graph, n, mix):
    say(f"radial lmax 3 U={U} graph={graph} n={n} mix={mix}")
    op, wl = _inputs(U, graph, n, seed=U + n)
    plan = tpc.Plan(_irreps(U), 3, 3, radial=(8, 64, RC), uvw=True)
    g = tpc.graph_build(T(wl.src), T(wl.dst), wl.n_nodes)
    rs = tpc.gather_rows(T(wl.r), g.perm)
    Y = tpc.sph_harm(3, rs)
    rl = tpc.gather_rows(T(wl.r_len), g.perm)
    x, W1, W2, go = T(wl.x), T(wl.W1), T(wl.W2), T(wl.g)
    Wm = T(wl.Wmix) if mix else None
    out, pre = tpc.forward_radial(plan, g, x, Y, rl, W1, W2, Wm)
    gx, gY, gW1, gW2, gWm, grl = tpc.backward_radial(plan, g, x, Y, rl, W1, W2, go, Wmix=Wm, out_pre=pre,
                                                     want=("x", "Y", "W1", "W2", "Wmix", "rlen"))
    out_r, pre_r = tpc.forward_radial_r(plan, g, x, rs, W1, W2, Wm)
    gx_r, gr_r, gW1_r, gW2_r, gWm_r = tpc.backward_radial_r(plan, g, x, rs, W1, W2, go, Wmix=Wm,
                                                            out_pre=pre_r)
    torch.cuda.synchronize()
    c = lambda t: None if t is None else t.cpu().numpy()
    p = c(g.perm)[:wl.n_edges]
    Yo = oracle.sh_real(3, wl.r)
    Wmo = wl.Wmix if mix else None
    ref, ref_pre = oracle.tp_conv_radial_fwd(op, wl.src, wl.dst, wl.n_nodes, wl.x, Yo, wl.r_len, wl.W1,
                                             wl.W2, wl.Wmix, 8, RC, return_pre_mix=True)
    want_out = ref if mix else ref_pre
    for o in (out, out_r):
        assert block_err(c(o), want_out, out_blocks(op)) <= TOL
    if mix:
        for q in (pre, pre_r):
            assert block_err(c(q), ref_pre, out_blocks(op)) <= TOL
    rb = oracle.tp_conv_radial_bwd(op, wl.src, wl.dst, wl.n_nodes, wl.x, Yo, wl.r_len, wl.W1, wl.W2, Wmo,
                                   wl.g, 8, RC, with_grad_rlen=True)
    for a in (gx, gx_r):
        assert block_err(c(a), rb[0], in_blocks(op)) <= TOL
    assert block_err(c(gY), rb[1][p], y_blocks(op)) <= TOL
    assert _vec_err(c(grl), rb[5][p]) <= TOL
    assert _vec_err(c(gr_r), _forces_ref(wl.r, rb[1], rb[5])[p]) <= TOL
    for res in (dict(gW1=c(gW1), gW2=c(gW2), gWm=c(gWm)), dict(gW1=c(gW1_r), gW2=c(gW2_r), gWm=c(gWm_r))):
        _check_params(op, res, rb, U)
    if not mix:
        assert gWm is None and gWm_r is None


def test_radial_l3_empty_and_isolated(tpc):
    """a graph with no edges (outputs zero, parameter gradients zero) and one
    whose last nodes receive and send nothing"""
    say("radial lmax 3 empty graph and isolated nodes")
    U = 16
    op = oracle.build_plan(_irreps(U), 3, 3)
    plan = tpc.Plan(_irreps(U), 3, 3, radial=(8, 64, RC))
    wl = make_workload("stream", dims_of(op), seed=5, n_nodes=40)
    gw = make_workload("lmax3", dims_of(op), seed=5, n_nodes=30, graph_only=True)
    for src, dst, r in ((np.zeros(0, np.int32), np.zeros(0, np.int32), np.zeros((0, 3), np.float32)),
                        (gw.src, gw.dst, gw.r)):
        g = tpc.graph_build(T(src), T(dst), 40)
        rs = tpc.gather_rows(T(r), g.perm)
        Y = tpc.sph_harm(3, rs)
        rl = tpc.gather_rows(T(np.linalg.norm(r.astype(np.float64), axis=1).astype(np.float32)), g.perm)
        out, _ = tpc.forward_radial(plan, g, T(wl.x), Y, rl, T(wl.W1), T(wl.W2))
        gx, gY, gW1, gW2, _, _ = tpc.backward_radial(plan, g, T(wl.x), Y, rl, T(wl.W1), T(wl.W2), T(wl.g))
        torch.cuda.synchronize()
        Yo = oracle.sh_real(3, r) if len(src) else np.zeros((0, 16))
        ref = oracle.tp_conv_radial_fwd(op, src, dst, 40, wl.x, Yo, np.linalg.norm(r.astype(np.float64), axis=1),
                                        wl.W1, wl.W2, None, 8, RC)
        rb = oracle.tp_conv_radial_bwd(op, src, dst, 40, wl.x, Yo, np.linalg.norm(r.astype(np.float64), axis=1),
                                       wl.W1, wl.W2, None, wl.g, 8, RC)
        if len(src) == 0:
            for a in (out, gx, gW1, gW2):
                assert not torch.any(a != 0)
            continue
        assert block_err(out.cpu().numpy(), ref, out_blocks(op)) <= TOL
        assert not torch.any(out[30:] != 0) and not torch.any(gx[30:] != 0)
        assert block_err(gx.cpu().numpy(), rb[0], in_blocks(op)) <= TOL
        _check_params(op, dict(gW1=gW1.cpu().numpy(), gW2=gW2.cpu().numpy(), gWm=None),
                      (None, None, rb[2], rb[3], None), U)



def test_radial_l3_determinism(tpc):
    """two backward calls give bitwise equal gradients (fixed-order sums of the
    per-wave and per-workgroup partials)"""
    say("radial lmax 3 determinism")
    U = 32
    op, wl = _inputs(U, "zipf", 600, seed=11)
    plan = tpc.Plan(_irreps(U), 3, 3, radial=(8, 64, RC), uvw=True)
    g = tpc.graph_build(T(wl.src), T(wl.dst), wl.n_nodes)
    rs = tpc.gather_rows(T(wl.r), g.perm)
    Y = tpc.sph_harm(3, rs)
    rl = tpc.gather_rows(T(wl.r_len), g.perm)
    args = (plan, g, T(wl.x), Y, rl, T(wl.W1), T(wl.W2), T(wl.g))
    want = ("x", "Y", "W1", "W2", "Wmix", "rlen")
    _, pre = tpc.forward_radial(plan, g, T(wl.x), Y, rl, T(wl.W1), T(wl.W2), T(wl.Wmix))
    a = tpc.backward_radial(*args, Wmix=T(wl.Wmix), out_pre=pre, want=want)
    b = tpc.backward_radial(*args, Wmix=T(wl.Wmix), out_pre=pre, want=want)
    torch.cuda.synchronize()
    for s, t in zip(a, b):
        assert torch.equal(s, t)


@pytest.mark.parametrize("U,graph,n,mix,only", [(16, "zipf", 300, False, None), (64, "lmax3", 120, True, None),
                                                (32, "stream", 150, True, "r"), (16, "lmax3", 1100, True, None)])
def test_radial_l3_double_backward_parity(tpc, U, graph, n, mix, only):
    from tests.test_gpu_radial_double import _check, _cotangents, _gpu_dbl, _ref
    say(f"radial lmax 3 double bwd U={U} graph={graph} n={n} mix={mix} only={only}")
    op, wl = _inputs(U, graph, n, seed=U + 3 * n)
    plan = tpc.Plan(_irreps(U), 3, 3, radial=(8, 64, RC), uvw=True)
    ggx, ggY, ggr = _cotangents(op, wl.n_nodes, wl.n_edges, U + n)
    if only == "r":                                  # the weights' tangent alone
        ggx, ggY = None, None
    res = _gpu_dbl(tpc, plan, wl, mix, wl.g, ggx, ggY, ggr, lmax=3)
    ref = _ref(op, wl, mix, wl.g, ggx, ggY, ggr, lmax=3)
    _check(op, res, ref, U, res["perm"])
    if not mix:
        assert res["dWm"] is None
