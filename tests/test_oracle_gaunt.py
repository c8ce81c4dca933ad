"""Pins for the oracle of the Gaunt (spherical-grid) convolution.

The quadrature against closed-form monomial integrals; the Gaunt coefficients
against the pointwise product of two band-limited signals evaluated at random
directions (off any grid), the identity of degree 0, their permutation
symmetry and selection rules, and the Clebsch-Gordan closed form; the whole
convolution against a brute-force sum of pointwise products at random
directions, rotation and inversion equivariance, the degree-0 filter as a
sparse matrix product, and truncation in lmax_out."""
import math

import numpy as np
import pytest
import scipy.sparse

import oracle
from oracle.gaunt import gaunt_coefficients, gaunt_conv_bwd, gaunt_conv_fwd, gaunt_plan, sphere_quadrature
from tests._common import haar
from workloads import make_gaunt_weights, make_workload


def _sphere_monomial(a, b, c):
    """closed form of the integral of x^a y^b z^c over the unit sphere"""
    if a % 2 or b % 2 or c % 2:
        return 0.0
    g = math.gamma
    return 2 * g((a + 1) / 2) * g((b + 1) / 2) * g((c + 1) / 2) / g((a + b + c + 3) / 2)


@pytest.mark.parametrize("degree", [0, 1, 4, 6, 9])
def test_quadrature_integrates_monomials_exactly(degree):
    pts, wts = sphere_quadrature(degree)
    for a in range(degree + 1):
        for b in range(degree + 1 - a):
            for c in range(degree + 1 - a - b):
                got = float(np.sum(wts * pts[:, 0] ** a * pts[:, 1] ** b * pts[:, 2] ** c))
                assert abs(got - _sphere_monomial(a, b, c)) <= 1e-13


def test_quadrature_is_not_exact_beyond_its_degree():
    # a degree-4 rule must miss z^6 or (x^2 - y^2)^3-type azimuthal content
    pts, wts = sphere_quadrature(4)
    z6 = float(np.sum(wts * pts[:, 2] ** 6))
    assert abs(z6 - _sphere_monomial(0, 0, 6)) > 1e-6


def _coeffs_to_values(lmax, coef, s):
    return sh_values(lmax, s) @ coef


def sh_values(lmax, s):
    return oracle.sh_real(lmax, s)


@pytest.mark.parametrize("seed", [0, 1])
def test_gaunt_expansion_reproduces_pointwise_product(seed):
    rng = np.random.default_rng(seed)
    L1, L2 = 2, 3
    a = rng.normal(size=(L1 + 1) ** 2)
    b = rng.normal(size=(L2 + 1) ** 2)
    h = np.zeros((L1 + L2 + 1) ** 2)
    for l1 in range(L1 + 1):
        for l2 in range(L2 + 1):
            for l3 in range(L1 + L2 + 1):
                G = gaunt_coefficients(l1, l2, l3)
                h[l3 * l3:(l3 + 1) ** 2] += np.einsum("abc,a,b->c", G, a[l1 * l1:(l1 + 1) ** 2],
                                                     b[l2 * l2:(l2 + 1) ** 2])
    s = rng.normal(size=(60, 3))
    want = _coeffs_to_values(L1, a, s) * _coeffs_to_values(L2, b, s)
    got = _coeffs_to_values(L1 + L2, h, s)
    assert np.max(np.abs(got - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))


@pytest.mark.parametrize("l", [0, 1, 2, 3])
def test_gaunt_degree_zero_is_identity(l):
    n = 2 * l + 1
    assert np.max(np.abs(gaunt_coefficients(0, l, l)[0] - np.eye(n))) <= 1e-14
    assert np.max(np.abs(gaunt_coefficients(l, 0, l)[:, 0, :] - np.eye(n))) <= 1e-14
    assert np.max(np.abs(gaunt_coefficients(l, l, 0)[:, :, 0] - np.eye(n))) <= 1e-14


def test_gaunt_symmetry_and_selection_rules():
    for l1 in range(4):
        for l2 in range(4):
            for l3 in range(7):
                G = gaunt_coefficients(l1, l2, l3)
                if (l1 + l2 + l3) % 2 or l3 < abs(l1 - l2) or l3 > l1 + l2:
                    assert not np.any(G), (l1, l2, l3)
                    continue
                assert np.any(G)
                assert np.max(np.abs(G - gaunt_coefficients(l2, l1, l3).transpose(1, 0, 2))) <= 1e-14
                assert np.max(np.abs(G - gaunt_coefficients(l3, l2, l1).transpose(2, 1, 0))) <= 1e-14


def test_gaunt_matches_clebsch_gordan_closed_form():
    """(1/4pi) int Y_a Y_b Y_c = sqrt((2l1+1)(2l2+1)/(2l3+1)) <l1 0 l2 0|l3 0> C_real[a,b,c]
    up to the sign convention of the real CG tensor (one sign per triple)."""
    for l1 in range(4):
        for l2 in range(4):
            for l3 in range(abs(l1 - l2), l1 + l2 + 1):
                if (l1 + l2 + l3) % 2:
                    continue
                G = gaunt_coefficients(l1, l2, l3)
                C = oracle.cg_real(l1, l2, l3)
                k = math.sqrt((2 * l1 + 1) * (2 * l2 + 1) / (2 * l3 + 1)) * \
                    oracle.cg_complex(l1, 0, l2, 0, l3, 0)
                ref = k * C
                i = np.unravel_index(np.argmax(np.abs(ref)), ref.shape)
                sgn = np.sign(G[i] * ref[i])
                assert sgn != 0
                assert np.max(np.abs(G - sgn * ref)) <= 1e-13, (l1, l2, l3)


def _case(n=24, U=3, lsh=2, lout=2, seed=0, irreps=None):
    irreps = irreps or f"{U}x0e+{U}x1o+{U}x2e"
    gp = gaunt_plan(irreps, lsh, lout)
    wl = make_workload("mid", dict(xdim=gp.xdim, n_paths=1, U=U, outdim=gp.outdim,
                                   n_out_irreps=lout + 1), seed=seed, n_nodes=n)
    w = make_gaunt_weights(wl.n_edges, lsh, U, seed=seed)
    return gp, wl, oracle.sh_real(lsh, wl.r), w


def test_conv_equals_sum_of_pointwise_products_at_random_directions():
    # with lmax_out = 2 + 2 the projection is exact, so the output signal of each
    # receiver is the sum over its edges of f_sender * g_edge, pointwise
    gp, wl, Y, w = _case(n=10, lout=4)
    out = gaunt_conv_fwd(gp, wl.src, wl.dst, wl.n_nodes, wl.x, Y, w)
    rng = np.random.default_rng(5)
    s = rng.normal(size=(40, 3))
    Ys = sh_values(4, s)                                    # [S, 25]
    U = gp.U
    x = wl.x.astype(np.float64)
    want = np.zeros((wl.n_nodes, U, len(s)))
    for e in range(wl.n_edges):
        j, i = wl.src[e], wl.dst[e]
        f = np.zeros((U, len(s)))
        for l1, off in zip(gp.degrees, gp.in_offsets):
            xa = x[j, off:off + U * (2 * l1 + 1)].reshape(U, 2 * l1 + 1)
            f += xa @ Ys[:, l1 * l1:(l1 + 1) ** 2].T
        g = np.zeros((U, len(s)))
        for l2 in range(gp.lmax_sh + 1):
            z = Ys[:, l2 * l2:(l2 + 1) ** 2] @ Y[e, l2 * l2:(l2 + 1) ** 2]    # [S]
            g += w[e, l2, :, None].astype(np.float64) * z[None, :]
        want[i] += f * g
    got = np.zeros_like(want)
    for l3 in range(5):
        o = gp.out_offsets[l3]
        blk = out[:, o:o + U * (2 * l3 + 1)].reshape(wl.n_nodes, U, 2 * l3 + 1)
        got += blk @ Ys[:, l3 * l3:(l3 + 1) ** 2].T
    assert np.max(np.abs(got - want)) <= 1e-11 * max(1.0, np.max(np.abs(want)))


def _rotate_blocks(arr, U, degs, offs, R, inversion=False):
    arr = np.array(arr, dtype=np.float64)
    for l, off in zip(degs, offs):
        s = slice(off, off + U * (2 * l + 1))
        blk = arr[:, s].reshape(arr.shape[0], U, 2 * l + 1)
        blk = blk * (-1) ** l if inversion else blk @ oracle.wigner_D_real(l, R).T
        arr[:, s] = blk.reshape(arr.shape[0], -1)
    return arr


def test_conv_rotation_and_inversion_equivariance():
    gp, wl, Y, w = _case(n=30)
    out = gaunt_conv_fwd(gp, wl.src, wl.dst, wl.n_nodes, wl.x, Y, w)
    odeg = list(range(gp.lmax_out + 1))
    R = haar(np.random.default_rng(3))
    xr = _rotate_blocks(wl.x, gp.U, gp.degrees, gp.in_offsets, R)
    Yr = oracle.sh_real(gp.lmax_sh, wl.r.astype(np.float64) @ R.T)
    got = gaunt_conv_fwd(gp, wl.src, wl.dst, wl.n_nodes, xr, Yr, w)
    want = _rotate_blocks(out, gp.U, odeg, gp.out_offsets, R)
    assert np.max(np.abs(got - want)) <= 1e-10 * max(1.0, np.max(np.abs(out)))
    xi = _rotate_blocks(wl.x, gp.U, gp.degrees, gp.in_offsets, None, inversion=True)
    Yi = oracle.sh_real(gp.lmax_sh, -wl.r.astype(np.float64))
    got = gaunt_conv_fwd(gp, wl.src, wl.dst, wl.n_nodes, xi, Yi, w)
    want = _rotate_blocks(out, gp.U, odeg, gp.out_offsets, None, inversion=True)
    assert np.max(np.abs(got - want)) <= 1e-10 * max(1.0, np.max(np.abs(out)))


def test_degree_zero_filter_is_a_sparse_matrix_product():
    gp, wl, Y, w = _case(n=20)
    w = np.array(w, dtype=np.float64)
    w[:, 1:, :] = 0.0
    out = gaunt_conv_fwd(gp, wl.src, wl.dst, wl.n_nodes, wl.x, Y, w)
    U = gp.U
    for l, off in zip(gp.degrees, gp.in_offsets):
        d = 2 * l + 1
        xb = wl.x[:, off:off + U * d].astype(np.float64).reshape(-1, U, d)
        want = np.zeros((wl.n_nodes, U, d))
        for u in range(U):
            A = scipy.sparse.csr_matrix((w[:, 0, u], (wl.dst, wl.src)), shape=(wl.n_nodes,) * 2)
            want[:, u, :] = A @ xb[:, u, :]
        o = gp.out_offsets[l]
        got = out[:, o:o + U * d].reshape(-1, U, d)
        assert np.max(np.abs(got - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))


def test_lower_lmax_out_is_a_prefix():
    gp4, wl, Y, w = _case(n=16, lout=4)
    gp2 = gaunt_plan(f"{gp4.U}x0e+{gp4.U}x1o+{gp4.U}x2e", 2, 2)
    o4 = gaunt_conv_fwd(gp4, wl.src, wl.dst, wl.n_nodes, wl.x, Y, w)
    o2 = gaunt_conv_fwd(gp2, wl.src, wl.dst, wl.n_nodes, wl.x, Y, w)
    assert np.max(np.abs(o4[:, :gp2.outdim] - o2)) <= 1e-13 * max(1.0, np.max(np.abs(o2)))


def test_plan_rejects_bad_irreps():
    with pytest.raises(ValueError):
        gaunt_plan("4x0e+4x1e", 2, 2)
    with pytest.raises(ValueError):
        gaunt_plan("4x0e+8x1o", 2, 2)
    with pytest.raises(ValueError):
        gaunt_plan("4x1o+4x1o", 2, 2)


def test_backward_trilinearity():
    # out is linear in each of x, Y, w: <g, out> = <grad_x, x> = <grad_Y, Y> = <grad_w, w>
    gp, wl, Y, w = _case(n=20, seed=2)
    rng = np.random.default_rng(9)
    g = rng.normal(size=(wl.n_nodes, gp.outdim))
    out = gaunt_conv_fwd(gp, wl.src, wl.dst, wl.n_nodes, wl.x, Y, w)
    gx, gY, gw = gaunt_conv_bwd(gp, wl.src, wl.dst, wl.n_nodes, wl.x, Y, w, g)
    ref = float(np.sum(g * out))
    for got in (np.sum(gx * wl.x), np.sum(gY * Y), np.sum(gw * np.asarray(w, dtype=np.float64))):
        assert abs(float(got) - ref) <= 1e-12 * max(1.0, abs(ref))


def test_backward_central_differences():
    gp, wl, Y, w = _case(n=6, U=2, seed=3)
    w = np.asarray(w, dtype=np.float64)
    rng = np.random.default_rng(4)
    g = rng.normal(size=(wl.n_nodes, gp.outdim))
    x = wl.x.astype(np.float64)
    gx, gY, gw = gaunt_conv_bwd(gp, wl.src, wl.dst, wl.n_nodes, x, Y, w, g)
    f = lambda x_, Y_, w_: float(np.sum(g * gaunt_conv_fwd(gp, wl.src, wl.dst, wl.n_nodes, x_, Y_, w_)))
    h = 1e-6
    for arr, grad, name in ((x, gx, "x"), (Y, gY, "Y"), (w, gw, "w")):
        flat = arr.reshape(-1)
        for k in rng.choice(flat.size, size=min(12, flat.size), replace=False):
            d = np.zeros_like(flat)
            d[k] = h
            args = {"x": x, "Y": Y, "w": w}
            args[name] = (flat + d).reshape(arr.shape)
            fp = f(args["x"], args["Y"], args["w"])
            args[name] = (flat - d).reshape(arr.shape)
            fm = f(args["x"], args["Y"], args["w"])
            num = (fp - fm) / (2 * h)
            assert abs(num - grad.reshape(-1)[k]) <= 1e-7 * max(1.0, abs(num)), (name, k)


def test_double_backward_by_differences_and_multilinearity():
    """The second-order backward: central differences of the first backward's
    loss L = <ggx, gx> + <ggY, gY> + <ggw, gw> in each of x, Y, w and g (exact
    up to rounding: every term is multilinear), <dg, g> = L, and missing
    cotangents as zeros."""
    from oracle.gaunt import gaunt_conv_double_bwd
    gp, wl, Y, w = _case(n=10, U=3, seed=5)
    w = np.asarray(w, dtype=np.float64).reshape(wl.n_edges, gp.lmax_sh + 1, gp.U)
    rng = np.random.default_rng(6)
    x = wl.x.astype(np.float64)
    g = rng.normal(size=(wl.n_nodes, gp.outdim))
    args = (gp, wl.src, wl.dst, wl.n_nodes)
    cot = [rng.normal(size=a.shape) for a in (x, Y, w)]

    def L(x_, Y_, w_, g_):
        return float(sum(np.sum(c * v) for c, v in zip(cot, gaunt_conv_bwd(*args, x_, Y_, w_, g_))))

    dx, dY, dw, dg = gaunt_conv_double_bwd(*args, x, Y, w, g, *cot)
    h = 1e-3
    base = [x, Y, w, g]
    for which, grad in enumerate((dx, dY, dw, dg)):
        d = rng.normal(size=base[which].shape)
        up, dn = list(base), list(base)
        up[which] = base[which] + h * d
        dn[which] = base[which] - h * d
        fd = (L(*up) - L(*dn)) / (2 * h)
        an = float(np.sum(grad * d))
        assert abs(fd - an) <= 1e-9 * max(1.0, abs(an)), which
    Lv = L(x, Y, w, g)
    assert abs(float(np.sum(dg * g)) - Lv) <= 1e-10 * max(1.0, abs(Lv))
    a = gaunt_conv_double_bwd(*args, x, Y, w, g, cot[0], None, None)
    b = gaunt_conv_double_bwd(*args, x, Y, w, g, cot[0], np.zeros_like(Y), np.zeros_like(w))
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
