"""GPU parity of the edge-vector form (tp_conv_forward_r / tp_conv_backward_r):
the harmonics are evaluated inside the convolution kernels from r [E][3] and
the backward returns grad_r = sum_b grad_Y[b] dY_b/dr without storing grad_Y.

Against the float64 oracle (harmonics, product and the harmonics' Jacobian of
its own) within 1e-4 x max|ref| per block, and against the library's Y form
(tp_conv_sph_harm + tp_conv_forward / tp_conv_backward), which evaluates the
same float32 harmonics: out, grad_x and grad_w must then be identical bit for
bit, grad_r equal to tp_conv_sph_harm_backward of grad_Y up to summation order.
"""
import numpy as np
import pytest

import oracle
from tests._common import dims_of
from tests.test_gpu_parity import (T, TOL, _sample, block_err, in_blocks, out_blocks, plans, say,
                                   w_err)
from workloads import make_workload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tpc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tensor_product_convolution_amd as m
    m.lib()
    return m


def run_geom(tpc, plan, wl, want=("x", "r", "w"), with_y_form=False):
    g = tpc.graph_build(T(wl.src), T(wl.dst), wl.n_nodes)
    r = tpc.gather_rows(T(wl.r), g.perm)
    w = tpc.gather_rows(T(wl.w), g.perm)
    x, go = T(wl.x), T(wl.g)
    res = dict(out=tpc.forward_r(plan, g, x, r, w))
    res["gx"], res["gr"], res["gw"] = tpc.backward_r(plan, g, x, r, w, go, want=want)
    if with_y_form:
        Y = tpc.sph_harm(plan.lmax_sh, r)
        res["out_y"] = tpc.forward(plan, g, x, Y, w)
        res["gx_y"], gY, res["gw_y"] = tpc.backward(plan, g, x, Y, w, go)
        res["gr_y"] = tpc.sph_harm_backward(plan.lmax_sh, r, gY)
    torch.cuda.synchronize()
    res = {k: (None if v is None else v.cpu().numpy()) for k, v in res.items()}
    res["perm"] = g.perm.cpu().numpy()[:wl.n_edges]
    return res


def _vec_err(got, ref):
    return float(np.max(np.abs(got - ref)) / max(float(np.max(np.abs(ref))), 1e-30))


@pytest.mark.parametrize("name,n_nodes,mul", [
    ("tiny", None, None),
    ("mid", None, None),
    ("lmax3", 400, None),
    ("zipf", 500, None),
    ("mid", 200, 8),
    ("mid", 1100, 16),       # past the small-graph launch threshold
    ("mid", 200, 64),
    ("lmax3", 150, 32),
    ("lmax3", 100, 128),
    ("tiny", None, 16),
])
def test_geom_parity(tpc, name, n_nodes, mul):
    say(f"edge-vector form parity {name} n={n_nodes} mul={mul}")
    plan, op = plans(name, mul)
    wl = make_workload(name, dims_of(op), n_nodes=n_nodes)
    res = run_geom(tpc, plan, wl)
    Y = oracle.sh_real(op.lmax_sh, wl.r)
    ref = oracle.tp_conv_fwd(op, wl.src, wl.dst, wl.n_nodes, wl.x, Y, wl.w)
    assert block_err(res["out"], ref, out_blocks(op)) <= TOL
    gx, gY, gw = oracle.tp_conv_bwd(op, wl.src, wl.dst, wl.n_nodes, wl.x, Y, wl.w, wl.g)
    p = res["perm"]
    assert block_err(res["gx"], gx, in_blocks(op)) <= TOL
    assert w_err(res["gw"], gw[p]) <= TOL
    gr = oracle.sh_real_vjp(op.lmax_sh, wl.r.astype(np.float64), gY)[p]
    assert _vec_err(res["gr"], gr) <= TOL


@pytest.mark.parametrize("name", ["mid", "lmax3"])
@pytest.mark.parametrize("want", [("r",), ("x",), ("w",), ("x", "r"), ("w", "r"), ("x", "w")])
def test_geom_output_subsets(tpc, name, want):
    """every subset of outputs: the one-pass backward (lmax 2, grad_x with an
    edge gradient) or the receiver and sender passes, each output as in the
    full call"""
    say(f"edge-vector form subsets {name} {want}")
    plan, op = plans(name)
    wl = make_workload(name, dims_of(op), n_nodes=300)
    full = run_geom(tpc, plan, wl)
    part = run_geom(tpc, plan, wl, want=want)
    for k, key in (("x", "gx"), ("r", "gr"), ("w", "gw")):
        if k in want:
            assert _vec_err(part[key], full[key]) <= 1e-6, key
        else:
            assert part[key] is None


@pytest.mark.parametrize("name", ["mid", "zipf"])
def test_geom_full_size_against_y_form_and_oracle(tpc, name):
    """Full-size 1,536-atom and Zipf graphs: the same float32 harmonics on both
    paths, so out, grad_x and grad_w are bit-identical to the Y form; grad_r
    agrees with tp_conv_sph_harm_backward of grad_Y; sampled rows against the
    oracle (receivers for out and grad_r, senders for grad_x)."""
    say(f"edge-vector form full size {name}")
    plan, op = plans(name)
    wl = make_workload(name, dims_of(op))
    res = run_geom(tpc, plan, wl, with_y_form=True)
    for a, b in (("out", "out_y"), ("gx", "gx_y"), ("gw", "gw_y")):
        assert np.array_equal(res[a], res[b]), a
    assert _vec_err(res["gr"], res["gr_y"]) <= 1e-5
    rng = np.random.default_rng(9)
    N = wl.n_nodes
    recv = _sample(np.bincount(wl.dst, minlength=N), 30, rng)
    e = np.nonzero(np.isin(wl.dst, recv))[0]
    Y = oracle.sh_real(op.lmax_sh, wl.r[e])
    ref = oracle.tp_conv_fwd(op, wl.src[e], wl.dst[e], N, wl.x, Y, wl.w[e])
    assert block_err(res["out"][recv], ref[recv], out_blocks(op)) <= TOL
    _, gY, _ = oracle.tp_conv_bwd(op, wl.src[e], wl.dst[e], N, wl.x, Y, wl.w[e], wl.g)
    inv = np.empty(wl.n_edges, np.int64)
    inv[res["perm"]] = np.arange(wl.n_edges)
    gr = oracle.sh_real_vjp(op.lmax_sh, wl.r[e].astype(np.float64), gY)
    assert _vec_err(res["gr"][inv[e]], gr) <= TOL
    send = _sample(np.bincount(wl.src, minlength=N), 30, rng)
    e2 = np.nonzero(np.isin(wl.src, send))[0]
    Y2 = oracle.sh_real(op.lmax_sh, wl.r[e2])
    gx, _, _ = oracle.tp_conv_bwd(op, wl.src[e2], wl.dst[e2], N, wl.x, Y2, wl.w[e2], wl.g)
    assert block_err(res["gx"][send], gx[send], in_blocks(op)) <= TOL


def test_geom_zero_vectors_and_empty_graph(tpc):
    """A zero edge vector has no direction: both forms evaluate the harmonics'
    formulas at the zero direction (x = y = z = 0) and give it a zero gradient;
    an empty graph gives zero outputs."""
    say("edge-vector form degenerate cases")
    plan, op = plans("mid")
    wl = make_workload("mid", dims_of(op), n_nodes=200)
    wl.r[::7] = 0.0
    res = run_geom(tpc, plan, wl, with_y_form=True)
    for a, b in (("out", "out_y"), ("gx", "gx_y"), ("gw", "gw_y")):
        assert np.array_equal(res[a], res[b]), a
    assert _vec_err(res["gr"], res["gr_y"]) <= 1e-5
    zero = np.nonzero(np.all(wl.r[res["perm"]] == 0, axis=1))[0]
    assert len(zero) > 0 and np.all(res["gr"][zero] == 0)
    N = 5
    g = tpc.graph_build(T(np.zeros(0, np.int32)), T(np.zeros(0, np.int32)), N)
    x = torch.randn(N, op.xdim, device="cuda:0")
    r = torch.zeros(0, 3, device="cuda:0")
    w = torch.zeros(0, op.n_paths, op.U, device="cuda:0")
    out = tpc.forward_r(plan, g, x, r, w)
    gx, gr, gw = tpc.backward_r(plan, g, x, r, w, torch.randn(N, op.outdim, device="cuda:0"))
    torch.cuda.synchronize()
    assert float(out.abs().max()) == 0.0 and float(gx.abs().max()) == 0.0
    assert gr.shape == (0, 3) and gw.shape[0] == 0


# ---------------------------------------------------------------------------
# the streaming radial layer from edge vectors


def _radial_geom(tpc, plan, wl, mix, g2, with_y_form=False):
    g = tpc.graph_build(T(wl.src), T(wl.dst), wl.n_nodes)
    r = tpc.gather_rows(T(wl.r), g.perm)
    x, W1, W2 = T(wl.x), T(wl.W1), T(wl.W2)
    Wm = T(wl.Wmix) if mix else None
    out, pre = tpc.forward_radial_r(plan, g, x, r, W1, W2, Wm)
    gx, gr, gW1, gW2, gWm = tpc.backward_radial_r(plan, g, x, r, W1, W2, T(g2), Wmix=Wm, out_pre=pre)
    res = dict(out=out, pre=pre, gx=gx, gr=gr, gW1=gW1, gW2=gW2, gWm=gWm)
    if with_y_form:
        Y = tpc.sph_harm(2, r)
        rl = tpc.gather_rows(T(wl.r_len), g.perm)
        o, p = tpc.forward_radial(plan, g, x, Y, rl, W1, W2, Wm)
        b = tpc.backward_radial(plan, g, x, Y, rl, W1, W2, T(g2), Wmix=Wm, out_pre=p,
                                want=("x", "Y", "W1", "W2", "Wmix", "rlen"))
        res.update(out_y=o, gx_y=b[0], gW1_y=b[2], gW2_y=b[3], gWm_y=b[4],
                   gr_y=tpc.sph_harm_backward(2, r, b[1], b[5]))
    torch.cuda.synchronize()
    res = {k: (None if v is None else v.cpu().numpy()) for k, v in res.items()}
    res["perm"] = g.perm.cpu().numpy()[:wl.n_edges]
    return res


@pytest.mark.parametrize("U,name,n,mix", [(16, "stream", 300, True), (128, "stream", 120, True),
                                          (16, "zipf", 400, False), (128, "lmax3", 100, True)])
def test_radial_geom_parity(tpc, U, name, n, mix):
    """forward and backward of the radial layer from r against the oracle: out,
    grad_x, the parameter gradients and grad_r through the harmonics and the
    lengths (the oracle's Jacobian of its harmonics and of |r|)"""
    from tests.test_gpu_radial import RC, _check_params, _forces_ref, _irreps, _radial_inputs
    say(f"radial edge-vector form U={U} graph={name} n={n} mix={mix}")
    op, wl = _radial_inputs(U, name, n)
    plan = tpc.Plan(_irreps(U), 2, 2, radial=(8, 64, RC), uvw=True)
    res = _radial_geom(tpc, plan, wl, mix, wl.g)
    Yo = oracle.sh_real(2, wl.r)
    out = oracle.tp_conv_radial_fwd(op, wl.src, wl.dst, wl.n_nodes, wl.x, Yo, wl.r_len, wl.W1, wl.W2,
                                    wl.Wmix if mix else None, 8, RC)
    assert block_err(res["out"], out, out_blocks(op)) <= TOL
    ref = oracle.tp_conv_radial_bwd(op, wl.src, wl.dst, wl.n_nodes, wl.x, Yo, wl.r_len, wl.W1, wl.W2,
                                    wl.Wmix if mix else None, wl.g, 8, RC, with_grad_rlen=True)
    assert block_err(res["gx"], ref[0], in_blocks(op)) <= TOL
    p = res["perm"]
    assert _vec_err(res["gr"], _forces_ref(wl.r, ref[1], ref[5])[p]) <= TOL
    _check_params(op, res, ref, U)


def test_radial_geom_full_size_against_y_form(tpc):
    """The 100,000-atom / 3,000,000-edge layer from r against the Y form (the
    harmonics and tp_conv_sph_harm_backward of grad_Y and grad_rlen): the same
    float32 harmonics, lengths from a float32 square root on chip against the
    given float32 lengths, so the results agree to float32 rounding."""
    from tests.test_gpu_radial import RC, _irreps
    say("radial edge-vector form full size")
    U = 128
    op = oracle.build_plan(_irreps(U), 2, 2)
    wl = make_workload("stream", dims_of(op))
    plan = tpc.Plan(_irreps(U), 2, 2, radial=(8, 64, RC), uvw=True)
    res = _radial_geom(tpc, plan, wl, True, wl.g, with_y_form=True)
    assert block_err(res["out"], res["out_y"], out_blocks(op)) <= 1e-5
    assert block_err(res["gx"], res["gx_y"], in_blocks(op)) <= 1e-5
    for k in ("gW1", "gW2", "gWm"):
        assert _vec_err(res[k], res[k + "_y"]) <= 1e-5, k
    assert _vec_err(res["gr"], res["gr_y"]) <= 1e-5
