"""Pins for the oracle of the fully connected per-edge-weight convolution:
reduction to the channel-wise product when every weight matrix is diagonal,
reduction to the channel mix when the weights do not depend on the edge,
rotation equivariance, and the multilinearity identities and central
differences of its backward."""
import numpy as np

import oracle
from oracle.fc import fc_conv_bwd, fc_conv_fwd
from tests._common import dims_of, haar
from tests.test_oracle_conv import _rotate_out, _rotate_x
from workloads import make_workload


def _case(irreps="4x0e+4x1o+4x2e", n=12, H=3, seed=0):
    plan = oracle.build_plan(irreps, 2, 2)
    wl = make_workload("mid", dims_of(plan), seed=seed, n_nodes=n)
    rng = np.random.default_rng(seed + 1)
    R = rng.normal(size=(wl.n_edges, H))
    Th = rng.normal(size=(H, plan.n_paths, plan.U, plan.U)) / plan.U
    return plan, wl, oracle.sh_real(2, wl.r), R, Th, rng


def test_diagonal_weights_reduce_to_channelwise_product():
    plan, wl, Y, R, _, rng = _case()
    th = rng.normal(size=(R.shape[1], plan.n_paths, plan.U))
    Th = np.einsum("hpu,uv->hpuv", th, np.eye(plan.U))
    got = fc_conv_fwd(plan, wl.src, wl.dst, wl.n_nodes, wl.x, Y, R, Th)
    w = np.einsum("eh,hpu->epu", R, th)
    want = oracle.tp_conv_fwd(plan, wl.src, wl.dst, wl.n_nodes, wl.x, Y, w)
    assert np.max(np.abs(got - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))


def test_edge_independent_weights_reduce_to_channel_mix():
    plan, wl, Y, _, _, rng = _case(H=1)
    R = np.ones((wl.n_edges, 1))
    K = len(plan.out_irreps)
    M = rng.normal(size=(K, plan.U, plan.U))
    Th = np.stack([M[plan.paths[p][4]] for p in range(plan.n_paths)])[None]   # [1, P, U, U]
    got = fc_conv_fwd(plan, wl.src, wl.dst, wl.n_nodes, wl.x, Y, R, Th)
    ones = np.ones((wl.n_edges, plan.n_paths, plan.U))
    want = oracle.uvw_mix_fwd(plan, oracle.tp_conv_fwd(plan, wl.src, wl.dst, wl.n_nodes, wl.x, Y, ones), M)
    assert np.max(np.abs(got - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))


def test_rotation_equivariance():
    plan, wl, Y, R, Th, _ = _case()
    out = fc_conv_fwd(plan, wl.src, wl.dst, wl.n_nodes, wl.x, Y, R, Th)
    Rm = haar(np.random.default_rng(3))
    Yr = oracle.sh_real(2, wl.r.astype(np.float64) @ Rm.T)
    got = fc_conv_fwd(plan, wl.src, wl.dst, wl.n_nodes, _rotate_x(plan, wl.x.astype(np.float64), Rm),
                      Yr, R, Th)
    assert np.max(np.abs(got - _rotate_out(plan, out, Rm))) <= 1e-10 * max(1.0, np.max(np.abs(out)))


def test_backward_multilinearity_and_differences():
    plan, wl, Y, R, Th, rng = _case()
    x = wl.x.astype(np.float64)
    g = rng.normal(size=(wl.n_nodes, plan.outdim))
    args = (plan, wl.src, wl.dst, wl.n_nodes)
    out = fc_conv_fwd(*args, x, Y, R, Th)
    f = float(np.sum(g * out))
    gx, gY, gR, gTh = fc_conv_bwd(*args, x, Y, R, Th, g)
    for grad, val in ((gx, x), (gY, Y), (gR, R), (gTh, Th)):
        assert abs(float(np.sum(grad * val)) - f) <= 1e-10 * max(1.0, abs(f))
    h = 1e-6
    for which in range(4):
        base = [x, Y, R, Th]
        d = rng.normal(size=base[which].shape)
        up, dn = list(base), list(base)
        up[which] = base[which] + h * d
        dn[which] = base[which] - h * d
        fd = (np.sum(g * fc_conv_fwd(*args, *up)) - np.sum(g * fc_conv_fwd(*args, *dn))) / (2 * h)
        an = float(np.sum([gx, gY, gR, gTh][which] * d))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an))


def test_double_backward_by_differences_and_multilinearity():
    """The second-order backward: central differences of the first backward's
    loss L = <ggx, gx> + <ggY, gY> + <ggR, gR> + <ggTheta, gTheta> in each of
    x, Y, R, Theta and g (exact up to rounding: every term is multilinear), the
    identity <dg, g> = L (L is linear in g), and missing cotangents as zeros."""
    from oracle.fc import fc_conv_double_bwd
    plan, wl, Y, R, Th, rng = _case(seed=4)
    x = wl.x.astype(np.float64)
    g = rng.normal(size=(wl.n_nodes, plan.outdim))
    args = (plan, wl.src, wl.dst, wl.n_nodes)
    cot = [rng.normal(size=a.shape) for a in (x, Y, R, Th)]

    def L(x_, Y_, R_, Th_, g_):
        return float(sum(np.sum(c * v) for c, v in zip(cot, fc_conv_bwd(*args, x_, Y_, R_, Th_, g_))))

    dx, dY, dR, dTh, dg = fc_conv_double_bwd(*args, x, Y, R, Th, g, *cot)
    h = 1e-3
    base = [x, Y, R, Th, g]
    for which, grad in enumerate((dx, dY, dR, dTh, dg)):
        d = rng.normal(size=base[which].shape)
        up, dn = list(base), list(base)
        up[which] = base[which] + h * d
        dn[which] = base[which] - h * d
        fd = (L(*up) - L(*dn)) / (2 * h)
        an = float(np.sum(grad * d))
        assert abs(fd - an) <= 1e-9 * max(1.0, abs(an)), which
    Lv = L(x, Y, R, Th, g)
    assert abs(float(np.sum(dg * g)) - Lv) <= 1e-10 * max(1.0, abs(Lv))
    a = fc_conv_double_bwd(*args, x, Y, R, Th, g, cot[0], None, None, None)
    b = fc_conv_double_bwd(*args, x, Y, R, Th, g, cot[0], np.zeros_like(Y), np.zeros_like(R),
                           np.zeros_like(Th))
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
