"""Pins for the oracle's convolution, adjoint, radial MLP, uvw mix and CSR.

Nothing here re-types the oracle's formulas: the forward is checked by
rotation and inversion equivariance, by reductions to library routines
(sparse matrix products, dot and cross products) and by a brute-force loop
over nonzeros written against the CG tensors; the backward by the
trilinearity identity and finite differences; the radial basis by scipy's
spherical Bessel function; the mix by a Kronecker-product route; the CSR by
plain Python loops.
"""
import numpy as np
import pytest
import scipy.sparse as sp
from scipy.special import spherical_jn

import oracle
from tests._common import dims_of, haar
from workloads import make_workload


def _wl(name, n_nodes=None, seed=0):
    cfg_irreps = {"tiny": ("8x0e+8x1o", 2, 2), "mid": ("32x0e+32x1o+32x2e", 2, 2),
                  "lmax3": ("64x0e+64x1o+64x2e+64x3o", 3, 3),
                  "zipf": ("64x0e+64x1o+64x2e+64x3o", 3, 3),
                  "stream": ("128x0e+128x1o+128x2e", 2, 2)}[name]
    plan = oracle.build_plan(*cfg_irreps)
    return plan, make_workload(name, dims_of(plan), seed=seed, n_nodes=n_nodes)


def _fwd(plan, wl, r=None, x=None, w=None):
    r = wl.r if r is None else r
    x = wl.x if x is None else x
    w = wl.w if w is None else w
    Y = oracle.sh_real(plan.lmax_sh, r)
    return oracle.tp_conv_fwd(plan, wl.src, wl.dst, wl.n_nodes, x, Y, w)


def _rotate_x(plan, x, R, inversion=False):
    x = np.array(x, dtype=np.float64)
    for (U, l, p), off in zip(plan.irreps_in, plan.in_offsets):
        s = slice(off, off + U * (2 * l + 1))
        blk = x[:, s].reshape(x.shape[0], U, 2 * l + 1)
        if inversion:
            blk = blk * p
        else:
            blk = blk @ oracle.wigner_D_real(l, R).T
        x[:, s] = blk.reshape(x.shape[0], -1)
    return x


def _rotate_out(plan, out, R, inversion=False):
    out = np.array(out)
    for (l, p), off in zip(plan.out_irreps, plan.out_offsets):
        s = slice(off, off + plan.U * (2 * l + 1))
        blk = out[:, s].reshape(out.shape[0], plan.U, 2 * l + 1)
        blk = blk * p if inversion else blk @ oracle.wigner_D_real(l, R).T
        out[:, s] = blk.reshape(out.shape[0], -1)
    return out


@pytest.mark.parametrize("name,n_nodes", [("tiny", None), ("mid", 96), ("lmax3", 64)])
def test_forward_rotation_and_inversion_equivariance(name, n_nodes):
    plan, wl = _wl(name, n_nodes)
    out = _fwd(plan, wl)
    tol = 1e-10 * max(1.0, float(np.max(np.abs(out))))
    R = haar(np.random.default_rng(11))
    got = _fwd(plan, wl, r=wl.r.astype(np.float64) @ R.T, x=_rotate_x(plan, wl.x, R))
    assert np.max(np.abs(got - _rotate_out(plan, out, R))) <= tol
    got = _fwd(plan, wl, r=-wl.r.astype(np.float64), x=_rotate_x(plan, wl.x, None, True))
    assert np.max(np.abs(got - _rotate_out(plan, out, None, True))) <= tol


def test_forward_brute_force_loop_tiny():
    plan, wl = _wl("tiny")
    Y = oracle.sh_real(plan.lmax_sh, wl.r)
    out = np.zeros((wl.n_nodes, plan.outdim))
    U = plan.U
    for e in range(wl.n_edges):
        j, i = int(wl.src[e]), int(wl.dst[e])
        for p, (ii, l1, l2, l3, k) in enumerate(plan.paths):
            C = oracle.cg_real(l1, l2, l3)
            for a, b, c in zip(*np.nonzero(C)):
                for u in range(U):
                    xv = wl.x[j, plan.in_offsets[ii] + u * (2 * l1 + 1) + a]
                    yv = Y[e, l2 * l2 + b]
                    out[i, plan.out_offsets[k] + u * (2 * l3 + 1) + c] += (
                        float(wl.w[e, p, u]) * C[a, b, c] * float(xv) * yv)
    assert np.max(np.abs(out - _fwd(plan, wl))) <= 1e-13


def _simple_graph(seed=5, n=40, e=300):
    rng = np.random.default_rng(seed)
    src = rng.integers(0, n, e)
    dst = rng.integers(0, n, e)
    r = rng.normal(size=(e, 3))
    return rng, n, src, dst, r


def test_reduction_000_is_sparse_matmul():
    plan = oracle.build_plan("6x0e", 0, 0)
    assert [(l1, l2, l3) for _, l1, l2, l3, _ in plan.paths] == [(0, 0, 0)]
    rng, n, src, dst, r = _simple_graph()
    x = rng.normal(size=(n, 6))
    w = rng.normal(size=(len(src), 1, 6))
    Y = oracle.sh_real(0, r)
    out = oracle.tp_conv_fwd(plan, src, dst, n, x, Y, w)
    for u in range(6):
        A = sp.coo_matrix((w[:, 0, u] * Y[:, 0], (dst, src)), shape=(n, n)).tocsr()
        assert np.max(np.abs(out[:, u] - A @ x[:, u])) <= 1e-13


def test_reduction_110_is_dot_product():
    plan = oracle.build_plan("4x1o", 1, 0)
    assert [(l1, l2, l3) for _, l1, l2, l3, _ in plan.paths] == [(1, 1, 0)]
    rng, n, src, dst, r = _simple_graph(6)
    x = rng.normal(size=(n, 12))
    w = rng.normal(size=(len(src), 1, 4))
    Y = oracle.sh_real(1, r)
    out = oracle.tp_conv_fwd(plan, src, dst, n, x, Y, w)
    want = np.zeros((n, 4))
    xs = x[src].reshape(-1, 4, 3)
    np.add.at(want, dst, w[:, 0, :] * np.einsum("eua,ea->eu", xs, Y[:, 1:4]) / np.sqrt(3))
    assert np.max(np.abs(out - want)) <= 1e-13


def test_reduction_111_is_cross_product():
    plan = oracle.build_plan("4x1o", 1, 1)
    names = [(l1, l2, l3) for _, l1, l2, l3, _ in plan.paths]
    p111 = names.index((1, 1, 1))
    rng, n, src, dst, r = _simple_graph(8)
    x = rng.normal(size=(n, 12))
    w = np.zeros((len(src), plan.n_paths, 4))
    w[:, p111, :] = rng.normal(size=(len(src), 4))
    Y = oracle.sh_real(1, r)
    out = oracle.tp_conv_fwd(plan, src, dst, n, x, Y, w)
    k = plan.paths[p111][4]
    assert plan.out_irreps[k] == (1, 1)
    blk = out[:, plan.out_offsets[k]:plan.out_offsets[k] + 12].reshape(n, 4, 3)
    P = [1, 2, 0]      # (x,y,z) -> (y,z,x); inverse [2, 0, 1]
    Q = [2, 0, 1]
    xs = x[src].reshape(-1, 4, 3)[:, :, Q]   # Cartesian
    yc = Y[:, 1:4][:, Q]
    cr = np.cross(xs, yc[:, None, :])[:, :, P] / np.sqrt(2.0)
    want = np.zeros((n, 4, 3))
    np.add.at(want, dst, w[:, p111, :, None] * cr)
    assert np.max(np.abs(blk - want)) <= 1e-13


def test_reduction_0ll_is_scaled_harmonics():
    plan = oracle.build_plan("3x0e", 2, 2)
    assert [(l1, l2, l3) for _, l1, l2, l3, _ in plan.paths] == [(0, 0, 0), (0, 1, 1), (0, 2, 2)]
    rng, n, src, dst, r = _simple_graph(9)
    x = rng.normal(size=(n, 3))
    w = rng.normal(size=(len(src), 3, 3))
    Y = oracle.sh_real(2, r)
    out = oracle.tp_conv_fwd(plan, src, dst, n, x, Y, w)
    for p, (_, _, l2, l3, k) in enumerate(plan.paths):
        want = np.zeros((n, 3, 2 * l3 + 1))
        msg = (w[:, p, :] * x[src])[:, :, None] * Y[:, None, l2 * l2:(l2 + 1) ** 2]
        np.add.at(want, dst, msg)
        got = out[:, plan.out_offsets[k]:plan.out_offsets[k] + 3 * (2 * l3 + 1)]
        assert np.max(np.abs(got.reshape(n, 3, -1) - want)) <= 1e-13


@pytest.mark.parametrize("name,n_nodes", [("tiny", None), ("mid", 48), ("lmax3", 40)])
def test_backward_trilinearity_and_finite_differences(name, n_nodes):
    plan, wl = _wl(name, n_nodes)
    x = wl.x.astype(np.float64)
    w = wl.w.astype(np.float64)
    Y = oracle.sh_real(plan.lmax_sh, wl.r)
    g = wl.g.astype(np.float64)
    args = (plan, wl.src, wl.dst, wl.n_nodes)
    out = oracle.tp_conv_fwd(*args, x, Y, w)
    gx, gY, gw = oracle.tp_conv_bwd(*args, x, Y, w, g)
    f = float(np.sum(g * out))
    for grad, val in ((gx, x), (gw, w), (gY, Y)):
        assert abs(np.sum(grad * val) - f) <= 1e-12 * max(1.0, abs(f)) * 10
    rng = np.random.default_rng(4)
    h = 1e-6
    for which in range(3):
        for _ in range(3):
            d = [np.zeros_like(x), np.zeros_like(Y), np.zeros_like(w)]
            d[which] = rng.normal(size=d[which].shape)

            def F(s):
                return float(np.sum(g * oracle.tp_conv_fwd(
                    *args, x + s * d[0], Y + s * d[1], w + s * d[2])))
            fd = (F(h) - F(-h)) / (2 * h)
            an = float(np.sum([gx, gY, gw][which] * d[which]))
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an))


def test_bessel_basis_against_scipy():
    r = np.linspace(0.8, 5.0, 50)
    B = oracle.bessel_basis(r, 8, 5.0)
    for n in range(1, 9):
        k = n * np.pi / 5.0
        want = np.sqrt(2.0 / 5.0) * k * spherical_jn(0, k * r)
        assert np.max(np.abs(B[:, n - 1] - want)) <= 1e-14
    assert np.max(np.abs(oracle.bessel_basis(np.array([5.0]), 8, 5.0))) <= 1e-14


def test_radial_mlp_gradients_finite_differences():
    rng = np.random.default_rng(2)
    r = rng.uniform(0.8, 5.0, 20)
    W1 = rng.normal(size=(8, 16)) / np.sqrt(8)
    W2 = rng.normal(size=(16, 12)) / 4
    G = rng.normal(size=(20, 12))
    w, cache = oracle.radial_mlp_fwd(r, W1, W2, 8, 5.0)
    g1, g2 = oracle.radial_mlp_bwd(G, cache, W2)
    # linear in W2: <G, w> = <g2, W2>
    assert abs(np.sum(G * w) - np.sum(g2 * W2)) <= 1e-12
    h = 1e-6
    for _ in range(4):
        d1 = rng.normal(size=W1.shape)
        fp = np.sum(G * oracle.radial_mlp_fwd(r, W1 + h * d1, W2, 8, 5.0)[0])
        fm = np.sum(G * oracle.radial_mlp_fwd(r, W1 - h * d1, W2, 8, 5.0)[0])
        an = np.sum(g1 * d1)
        assert abs((fp - fm) / (2 * h) - an) <= 1e-7 * max(1.0, abs(an))


def test_uvw_mix_against_kronecker_route_and_adjoint():
    plan = oracle.build_plan("5x0e+5x1o+5x2e", 2, 2)
    rng = np.random.default_rng(3)
    n = 7
    out = rng.normal(size=(n, plan.outdim))
    W = rng.normal(size=(len(plan.out_irreps), 5, 5))
    out2 = oracle.uvw_mix_fwd(plan, out, W)
    for k, (l, _) in enumerate(plan.out_irreps):
        d = 2 * l + 1
        s = slice(plan.out_offsets[k], plan.out_offsets[k] + 5 * d)
        K = np.kron(W[k].T, np.eye(d))          # acts on the flattened [U][2l+1] block
        assert np.max(np.abs(out2[:, s] - out[:, s] @ K.T)) <= 1e-13
    g2 = rng.normal(size=out2.shape)
    go, gW = oracle.uvw_mix_bwd(plan, out, W, g2)
    f = np.sum(g2 * out2)
    assert abs(np.sum(go * out) - f) <= 1e-12 * max(1, abs(f))
    assert abs(np.sum(gW * W) - f) <= 1e-12 * max(1, abs(f))


@pytest.mark.parametrize("irreps,lmax", [("4x0e+4x1o+4x2e", 2), ("3x0e+3x1o+3x2e+3x3o", 3)])
def test_radial_conv_equivariance_and_gradients(irreps, lmax):
    # the stream workload's structure with a narrow plan, for speed
    plan = oracle.build_plan(irreps, lmax, lmax)
    wl = make_workload("stream", dims_of(plan), seed=1, n_nodes=12)
    x = wl.x.astype(np.float64)
    Y = oracle.sh_real(lmax, wl.r)
    rl = wl.r_len.astype(np.float64)
    args = (plan, wl.src, wl.dst, wl.n_nodes)
    kw = dict(n_basis=wl.n_basis, r_cut=wl.r_cut)
    out = oracle.tp_conv_radial_fwd(*args, x, Y, rl, wl.W1, wl.W2, wl.Wmix, **kw)
    R = haar(np.random.default_rng(5))
    Yr = oracle.sh_real(lmax, wl.r.astype(np.float64) @ R.T)
    got = oracle.tp_conv_radial_fwd(*args, _rotate_x(plan, x, R), Yr, rl, wl.W1, wl.W2,
                                    wl.Wmix, **kw)
    assert np.max(np.abs(got - _rotate_out(plan, out, R))) <= 1e-10 * max(1, np.max(np.abs(out)))
    g = wl.g.astype(np.float64)
    gx, gY, gW1, gW2, gWm = oracle.tp_conv_radial_bwd(*args, x, Y, rl, wl.W1, wl.W2, wl.Wmix, g, **kw)
    f = float(np.sum(g * out))
    for grad, val in ((gx, x), (gY, Y), (gW2, wl.W2), (gWm, wl.Wmix)):
        assert abs(np.sum(grad * val.astype(np.float64)) - f) <= 1e-11 * max(1.0, abs(f))
    rng = np.random.default_rng(6)
    h = 1e-6
    W1 = wl.W1.astype(np.float64)
    for _ in range(3):
        d = rng.normal(size=W1.shape)
        F = [float(np.sum(g * oracle.tp_conv_radial_fwd(*args, x, Y, rl, W1 + s * d, wl.W2,
                                                           wl.Wmix, **kw))) for s in (h, -h)]
        an = float(np.sum(gW1 * d))
        assert abs((F[0] - F[1]) / (2 * h) - an) <= 1e-7 * max(1.0, abs(an))


def test_csr_against_loops():
    rng = np.random.default_rng(12)
    n, e = 23, 400
    src = rng.integers(0, n, e)
    dst = rng.integers(0, n, e)
    c = oracle.csr_build(src, dst, n)
    perm, rp = [], [0]
    for i in range(n):
        perm += [k for k in range(e) if dst[k] == i]
        rp.append(len(perm))
    assert list(c["perm"]) == perm and list(c["row_ptr"]) == rp
    assert list(c["col"]) == [int(src[k]) for k in perm]
    tp, trp = [], [0]
    for j in range(n):
        tp += [q for q in range(e) if src[perm[q]] == j]
        trp.append(len(tp))
    assert list(c["t_perm"]) == tp and list(c["t_row_ptr"]) == trp
    assert list(c["t_col"]) == [int(dst[perm[q]]) for q in tp]


def test_launch_order_against_loops_and_its_defining_properties():
    """Nodes by descending degree, ties by node id: built by a plain loop over
    degrees from the largest down, and checked as a permutation whose degrees
    never rise and whose ties keep node order (empty and isolated nodes too)."""
    rng = np.random.default_rng(13)
    for n, e in ((23, 400), (50, 60), (7, 0), (1, 5), (300, 3000)):
        src = rng.integers(0, n, e)
        dst = rng.integers(0, max(1, n // 3), e)         # many nodes without in-edges
        c = oracle.csr_build(src, dst, n)
        for ptr in (c["row_ptr"], c["t_row_ptr"]):
            deg = [int(ptr[i + 1] - ptr[i]) for i in range(n)]
            want = [i for d in range(max(deg), -1, -1) for i in range(n) if deg[i] == d]
            got = oracle.launch_order(ptr)
            assert list(got) == want
            assert sorted(got) == list(range(n))
            for k in range(n - 1):
                a, b = got[k], got[k + 1]
                assert deg[a] > deg[b] or (deg[a] == deg[b] and a < b)


def test_workload_shapes():
    plan, wl = _wl("mid")
    assert wl.n_edges == 46080 and wl.n_nodes == 1536
    assert np.all(np.bincount(wl.dst, minlength=1536) == 30)
    assert np.all(wl.src != wl.dst)
    key = wl.dst.astype(np.int64) * 1536 + wl.src
    assert len(np.unique(key)) == wl.n_edges
    L = np.linalg.norm(wl.r, axis=1)
    assert L.min() >= 0.8 - 1e-6 and L.max() <= 5.0 + 1e-6
    assert abs(float(np.std(wl.w)) - 1 / np.sqrt(15)) < 0.01
    plan, wl = _wl("tiny")
    assert np.all(np.linalg.norm(wl.r, axis=1) < 4.0)
    assert 300 < wl.n_edges < 800


def test_bessel_basis_derivative_against_scipy():
    r = np.linspace(0.8, 5.0, 50)
    dB = oracle.bessel_basis_deriv(r, 8, 5.0)
    for n in range(1, 9):
        k = n * np.pi / 5.0
        want = np.sqrt(2.0 / 5.0) * k * k * spherical_jn(0, k * r, derivative=True)
        assert np.max(np.abs(dB[:, n - 1] - want)) <= 1e-13


def _energy(fn, g):
    return float(np.sum(np.asarray(g, dtype=np.float64) * fn()))


def test_edge_vector_gradients_by_differences():
    """Forces: d<g, out>/dr through the harmonics (direct weights) and through
    the harmonics and the radial network (radial weights), by central
    differences of the forward in r."""
    rng = np.random.default_rng(9)
    h = 1e-6
    # direct weights: grad_r = J_Y^T grad_Y
    plan, wl = _wl("tiny")
    x = wl.x.astype(np.float64)
    w = wl.w.astype(np.float64)
    r = wl.r.astype(np.float64)
    g = wl.g.astype(np.float64)
    _, gY, _ = oracle.tp_conv_bwd(plan, wl.src, wl.dst, wl.n_nodes, x, oracle.sh_real(2, r), w, g)
    grad_r = oracle.sh_real_vjp(2, r, gY)
    for _ in range(3):
        d = rng.normal(size=r.shape)
        F = [_energy(lambda: oracle.tp_conv_fwd(plan, wl.src, wl.dst, wl.n_nodes, x,
                                                oracle.sh_real(2, r + s * d), w), g) for s in (h, -h)]
        an = float(np.sum(grad_r * d))
        assert abs((F[0] - F[1]) / (2 * h) - an) <= 1e-6 * max(1.0, abs(an))
    # radial weights with the mix: grad_r = J_Y^T grad_Y + grad_rlen r_hat
    plan = oracle.build_plan("4x0e+4x1o+4x2e", 2, 2)
    wl = make_workload("stream", dims_of(plan), seed=2, n_nodes=10)
    x, r, g = wl.x.astype(np.float64), wl.r.astype(np.float64), wl.g.astype(np.float64)
    kw = dict(n_basis=wl.n_basis, r_cut=wl.r_cut)
    args = (plan, wl.src, wl.dst, wl.n_nodes)
    rl = np.linalg.norm(r, axis=1)
    out = oracle.tp_conv_radial_bwd(*args, x, oracle.sh_real(2, r), rl, wl.W1, wl.W2, wl.Wmix, g,
                                    with_grad_rlen=True, **kw)
    gY, grl = out[1], out[5]
    grad_r = oracle.sh_real_vjp(2, r, gY) + grl[:, None] * r / rl[:, None]
    for _ in range(3):
        d = rng.normal(size=r.shape)
        F = []
        for s in (h, -h):
            rs = r + s * d
            F.append(_energy(lambda: oracle.tp_conv_radial_fwd(
                *args, x, oracle.sh_real(2, rs), np.linalg.norm(rs, axis=1), wl.W1, wl.W2,
                wl.Wmix, **kw), g))
        an = float(np.sum(grad_r * d))
        assert abs((F[0] - F[1]) / (2 * h) - an) <= 1e-6 * max(1.0, abs(an))
    # the length gradient alone, by differences in r_len at fixed directions
    Y = oracle.sh_real(2, r)
    d = rng.normal(size=rl.shape)
    F = [_energy(lambda: oracle.tp_conv_radial_fwd(*args, x, Y, rl + s * d, wl.W1, wl.W2, wl.Wmix,
                                                   **kw), g) for s in (h, -h)]
    an = float(np.sum(grl * d))
    assert abs((F[0] - F[1]) / (2 * h) - an) <= 1e-6 * max(1.0, abs(an))


def test_double_backward_by_differences_and_multilinearity():
    """The second-order backward: central differences of the first backward
    (exact up to rounding, every term being multilinear) in each of g, x, Y, w,
    and the scaling identities of a loss linear in g and affine in x, Y, w."""
    plan, wl = _wl("tiny")
    rng = np.random.default_rng(11)
    x, w, g = wl.x.astype(np.float64), wl.w.astype(np.float64), wl.g.astype(np.float64)
    Y = oracle.sh_real(2, wl.r)
    args = (plan, wl.src, wl.dst, wl.n_nodes)
    ggx, ggY, ggw = rng.normal(size=x.shape), rng.normal(size=Y.shape), rng.normal(size=w.shape)

    def L(x_, Y_, w_, g_):
        gx, gY, gw = oracle.tp_conv_bwd(*args, x_, Y_, w_, g_)
        return float(np.sum(ggx * gx) + np.sum(ggY * gY) + np.sum(ggw * gw))

    dx, dY, dw, dg = oracle.tp_conv_double_bwd(*args, x, Y, w, g, ggx, ggY, ggw)
    h = 1e-3
    for grad, name in ((dx, 0), (dY, 1), (dw, 2), (dg, 3)):
        base = [x, Y, w, g]
        d = rng.normal(size=base[name].shape)
        up = list(base)
        dn = list(base)
        up[name] = base[name] + h * d
        dn[name] = base[name] - h * d
        fd = (L(*up) - L(*dn)) / (2 * h)
        an = float(np.sum(grad * d))
        assert abs(fd - an) <= 1e-10 * max(1.0, abs(an))
    Lv = L(x, Y, w, g)
    assert abs(float(np.sum(dg * g)) - Lv) <= 1e-10 * max(1.0, abs(Lv))
    # L = F(g, ggx, Y, w) + F(g, x, ggY, w) + F(g, x, Y, ggw): the terms with x
    Fx = L(np.zeros_like(x), Y, w, g)
    assert abs(float(np.sum(dx * x)) - (Lv - Fx)) <= 1e-10 * max(1.0, abs(Lv))
    # missing cotangents are zeros
    a = oracle.tp_conv_double_bwd(*args, x, Y, w, g, ggx, None, None)
    b = oracle.tp_conv_double_bwd(*args, x, Y, w, g, ggx, np.zeros_like(Y), np.zeros_like(w))
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_bessel_second_derivative_against_the_spherical_bessel_equation():
    # B_n(r) = sqrt(2/r_c) k j0(k r): B_n'' = sqrt(2/r_c) k^3 j0''(k r), and j0
    # solves x^2 y'' + 2 x y' + x^2 y = 0, so j0'' = -j0 - 2 j0' / x
    r = np.linspace(0.8, 5.0, 50)
    d2B = oracle.bessel_basis_deriv2(r, 8, 5.0)
    for n in range(1, 9):
        k = n * np.pi / 5.0
        xx = k * r
        j0dd = -spherical_jn(0, xx) - 2.0 * spherical_jn(0, xx, derivative=True) / xx
        want = np.sqrt(2.0 / 5.0) * k ** 3 * j0dd
        assert np.max(np.abs(d2B[:, n - 1] - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))


def test_silu_derivatives_against_sympy():
    import sympy
    zs = sympy.Symbol("z")
    f = zs / (1 + sympy.exp(-zs))
    f1, f2 = sympy.diff(f, zs), sympy.diff(f, zs, 2)
    pts = np.array([-30.0, -4.5, -1.0, -0.3, 0.0, 0.7, 2.0, 6.0, 25.0])
    s0, s1, s2 = oracle.silu_derivs(pts)
    for i, p in enumerate(pts):
        for got, expr in ((s0[i], f), (s1[i], f1), (s2[i], f2)):
            want = float(expr.subs(zs, sympy.Float(p, 30)).evalf(30))
            assert abs(got - want) <= 1e-14 * max(1.0, abs(want))


def _radial_small(seed, n_nodes=10, lmax=2):
    irr = "4x0e+4x1o+4x2e" if lmax == 2 else "3x0e+3x1o+3x2e+3x3o"
    plan = oracle.build_plan(irr, lmax, lmax)
    wl = make_workload("stream", dims_of(plan), seed=seed, n_nodes=n_nodes)
    f64 = lambda a: np.asarray(a, dtype=np.float64)
    ins = dict(x=f64(wl.x), Y=oracle.sh_real(lmax, f64(wl.r)), r_len=f64(wl.r_len), W1=f64(wl.W1),
               W2=f64(wl.W2), Wmix=f64(wl.Wmix), g2=f64(wl.g))
    return plan, wl, ins


@pytest.mark.parametrize("with_mix,lmax", [(True, 2), (False, 2), (True, 3)])
def test_radial_double_backward_by_differences(with_mix, lmax):
    """Central differences of the first backward's loss in every input:
    L = <ggx, grad_x> + <ggY, grad_Y> + <ggr, grad_rlen> (the first backward
    is itself pinned by differences of the forward)."""
    plan, wl, ins = _radial_small(4, lmax=lmax)
    if not with_mix:
        ins["Wmix"] = None
    rng = np.random.default_rng(12)
    ggx = rng.normal(size=ins["x"].shape)
    ggY = rng.normal(size=ins["Y"].shape)
    ggr = rng.normal(size=ins["r_len"].shape)
    args = (plan, wl.src, wl.dst, wl.n_nodes)
    kw = dict(n_basis=wl.n_basis, r_cut=wl.r_cut)

    def L(v):
        o = oracle.tp_conv_radial_bwd(*args, v["x"], v["Y"], v["r_len"], v["W1"], v["W2"], v["Wmix"],
                                      v["g2"], with_grad_rlen=True, **kw)
        return float(np.sum(ggx * o[0]) + np.sum(ggY * o[1]) + np.sum(ggr * o[5]))

    dx, dY, drl, dW1, dW2, dWm, dg2 = oracle.tp_conv_radial_double_bwd(
        *args, ins["x"], ins["Y"], ins["r_len"], ins["W1"], ins["W2"], ins["Wmix"], ins["g2"],
        ggx=ggx, ggY=ggY, ggr=ggr, **kw)
    grads = dict(x=dx, Y=dY, r_len=drl, W1=dW1, W2=dW2, Wmix=dWm, g2=dg2)
    h = 1e-5
    for name, grad in grads.items():
        if ins[name] is None:
            assert grad is None
            continue
        for _ in range(2):
            d = rng.normal(size=ins[name].shape)
            if name == "r_len":
                d *= 0.1                        # stay inside the basis' range
            up, dn = dict(ins), dict(ins)
            up[name] = ins[name] + h * d
            dn[name] = ins[name] - h * d
            fd = (L(up) - L(dn)) / (2 * h)
            an = float(np.sum(grad * d))
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)


def test_radial_double_backward_without_length_cotangent_is_the_direct_one():
    """With no cotangent on grad_rlen the weight tangent vanishes: dx, dY and
    the (unmixed) d_g2 are the direct-weight second-order backward at
    w = network(r_len), and dW1, dW2 are the network's first backward of that
    pass's d_w."""
    plan, wl, ins = _radial_small(7)
    rng = np.random.default_rng(3)
    ggx, ggY = rng.normal(size=ins["x"].shape), rng.normal(size=ins["Y"].shape)
    args = (plan, wl.src, wl.dst, wl.n_nodes)
    kw = dict(n_basis=wl.n_basis, r_cut=wl.r_cut)
    dx, dY, drl, dW1, dW2, dWm, dg2 = oracle.tp_conv_radial_double_bwd(
        *args, ins["x"], ins["Y"], ins["r_len"], ins["W1"], ins["W2"], None, ins["g2"],
        ggx=ggx, ggY=ggY, **kw)
    w, cache = oracle.radial_mlp_fwd(ins["r_len"], ins["W1"], ins["W2"], wl.n_basis, wl.r_cut)
    w = w.reshape(wl.n_edges, plan.n_paths, plan.U)
    ex, eY, ew, eg = oracle.tp_conv_double_bwd(*args, ins["x"], ins["Y"], w, ins["g2"], ggx, ggY, None)
    gW1, gW2, gB = oracle.radial_mlp_bwd(ew.reshape(wl.n_edges, -1), cache, ins["W2"], ins["W1"])
    grl = np.sum(gB * oracle.bessel_basis_deriv(ins["r_len"], wl.n_basis, wl.r_cut), axis=1)
    for got, want in ((dx, ex), (dY, eY), (dg2, eg), (dW1, gW1), (dW2, gW2), (drl, grl)):
        assert np.allclose(got, want, rtol=1e-12, atol=1e-12)
    assert dWm is None


def test_radial_double_backward_is_linear_in_the_cotangents():
    plan, wl, ins = _radial_small(8)
    rng = np.random.default_rng(5)
    cot = dict(ggx=rng.normal(size=ins["x"].shape), ggY=rng.normal(size=ins["Y"].shape),
               ggr=rng.normal(size=ins["r_len"].shape))
    args = (plan, wl.src, wl.dst, wl.n_nodes, ins["x"], ins["Y"], ins["r_len"], ins["W1"], ins["W2"],
            ins["Wmix"], ins["g2"])
    kw = dict(n_basis=wl.n_basis, r_cut=wl.r_cut)
    both = oracle.tp_conv_radial_double_bwd(*args, **cot, **kw)
    parts = [oracle.tp_conv_radial_double_bwd(*args, **{k: v}, **kw) for k, v in cot.items()]
    twice = oracle.tp_conv_radial_double_bwd(*args, **{k: 2 * v for k, v in cot.items()}, **kw)
    for i in range(7):
        s = sum(p[i] for p in parts)
        assert np.allclose(both[i], s, rtol=1e-10, atol=1e-12)
        assert np.allclose(twice[i], 2 * both[i], rtol=1e-12, atol=1e-12)
    none = oracle.tp_conv_radial_double_bwd(*args, **kw)
    assert all(np.max(np.abs(a)) == 0 for a in none)
