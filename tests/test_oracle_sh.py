"""Pins for the oracle's real spherical harmonics and Wigner-D matrices.

Checked against scipy's complex harmonics, closed-form polynomials from the
standard table of real harmonics, the addition theorem, parity, quadrature
orthonormality, and sympy's Euler-angle Wigner-D.
"""
import numpy as np
import pytest
from scipy.special import sph_harm_y
from scipy.spatial.transform import Rotation as SciRot
from sympy.physics.quantum.spin import Rotation as SymRot

import oracle


def _dirs(n, seed=3):
    v = np.random.default_rng(seed).normal(size=(n, 3))
    return v / np.linalg.norm(v, axis=1, keepdims=True)


def test_complex_sh_matches_scipy():
    r = _dirs(200)
    theta = np.arccos(r[:, 2])
    phi = np.arctan2(r[:, 1], r[:, 0])
    for l in range(6):
        ours = oracle.sh_complex(l, r)
        for m in range(-l, l + 1):
            ref = sph_harm_y(l, m, theta, phi)
            assert np.max(np.abs(ours[:, m + l] - ref)) <= 1e-13


def test_real_sh_closed_forms():
    """Standard real harmonics times sqrt(4 pi) (component normalisation)."""
    r = _dirs(100)
    x, y, z = r[:, 0], r[:, 1], r[:, 2]
    s3, s5, s7, s15 = np.sqrt(3), np.sqrt(5), np.sqrt(7), np.sqrt(15)
    s42, s70, s105 = np.sqrt(42), np.sqrt(70), np.sqrt(105)
    want = np.stack([
        np.ones_like(x),
        s3 * y, s3 * z, s3 * x,
        s15 * x * y, s15 * y * z, s5 / 2 * (3 * z * z - 1), s15 * x * z, s15 / 2 * (x * x - y * y),
        s70 / 4 * y * (3 * x * x - y * y), s105 * x * y * z, s42 / 4 * y * (5 * z * z - 1),
        s7 / 2 * z * (5 * z * z - 3), s42 / 4 * x * (5 * z * z - 1),
        s105 / 2 * z * (x * x - y * y), s70 / 4 * x * (x * x - 3 * y * y),
    ], axis=1)
    got = oracle.sh_real(3, r * 2.7)  # length must not matter
    assert np.max(np.abs(got - want)) <= 1e-13


def test_real_sh_norm_parity_and_addition():
    r = _dirs(64)
    Y = oracle.sh_real(5, r)
    Yn = oracle.sh_real(5, -r)
    for l in range(6):
        s = slice(l * l, (l + 1) ** 2)
        assert np.max(np.abs(np.sum(Y[:, s] ** 2, axis=1) - (2 * l + 1))) <= 1e-12
        assert np.max(np.abs(Yn[:, s] - (-1) ** l * Y[:, s])) <= 1e-13
        # addition theorem: sum_m Y_lm(a) Y_lm(b) = (2l+1) P_l(a.b)
        a, b = r[:32], r[32:]
        lhs = np.sum(Y[:32, s] * Y[32:, s], axis=1)
        Pl = np.polynomial.legendre.legval(np.sum(a * b, axis=1), [0] * l + [1])
        assert np.max(np.abs(lhs - (2 * l + 1) * Pl)) <= 1e-12


def test_real_sh_orthonormal_by_quadrature():
    lmax = 4
    ct, wt = np.polynomial.legendre.leggauss(lmax + 2)
    nphi = 2 * lmax + 3
    phi = 2 * np.pi * np.arange(nphi) / nphi
    CT, PHI = np.meshgrid(ct, phi, indexing="ij")
    st = np.sqrt(1 - CT ** 2)
    r = np.stack([st * np.cos(PHI), st * np.sin(PHI), CT], axis=-1).reshape(-1, 3)
    w = (wt[:, None] * np.full(nphi, 2 * np.pi / nphi)[None, :]).reshape(-1)
    Y = oracle.sh_real(lmax, r)
    # component normalisation: the sphere average of Y_lm Y_l'm' is delta
    G = (Y * w[:, None]).T @ Y / (4 * np.pi)
    assert np.max(np.abs(G - np.eye(G.shape[0]))) <= 1e-12


def test_zero_vector_rejected():
    with pytest.raises(ValueError):
        oracle.sh_real(2, np.zeros((1, 3)))


def _haar(seed):
    return SciRot.random(random_state=seed).as_matrix()


def test_wigner_D_properties():
    R1, R2 = _haar(1), _haar(2)
    P = np.array([[0, 1, 0], [0, 0, 1], [1, 0, 0]], dtype=float)  # (x,y,z)->(y,z,x)
    for l in range(5):
        D1, res = oracle.wigner_D_real(l, R1, return_residual=True)
        assert res <= 1e-13
        D2 = oracle.wigner_D_real(l, R2)
        D12 = oracle.wigner_D_real(l, R1 @ R2)
        assert np.max(np.abs(D1 @ D1.T - np.eye(2 * l + 1))) <= 1e-12
        assert np.max(np.abs(D12 - D1 @ D2)) <= 1e-12
    assert np.max(np.abs(oracle.wigner_D_real(1, R1) - P @ R1 @ P.T)) <= 1e-12


def test_wigner_D_matches_sympy_euler_route():
    """sympy's D^l(alpha, beta, gamma) for R = Rz(a) Ry(b) Rz(g), moved to the real basis."""
    a, b, g = 0.3, 1.1, -0.7
    R = SciRot.from_euler("ZYZ", [a, b, g]).as_matrix()
    for l in range(4):
        Dc = np.array([[complex(SymRot.D(l, m, mp, a, b, g).doit().evalf())
                        for mp in range(-l, l + 1)] for m in range(-l, l + 1)])
        U = oracle.real_basis_matrix(l)
        # Y(R r) = conj(D) Y(r) for complex harmonics; real basis: U conj(D) U^H
        Dr = U @ Dc.conj() @ U.conj().T
        assert np.max(np.abs(Dr.imag)) <= 1e-12
        assert np.max(np.abs(Dr.real - oracle.wigner_D_real(l, R))) <= 1e-12


def test_sh_jacobian_against_differences_rotation_and_closed_form():
    """dY/dr: central differences of sh_real, zero along r (a function of the
    direction only), rotation covariance J(Rr) = D J(r) R^T, and the l = 1
    closed form sqrt3 (P - (P u) u^T) / |r| with P the (y, z, x) permutation."""
    rng = np.random.default_rng(8)
    r = rng.normal(size=(40, 3)) * rng.uniform(0.5, 3.0, size=(40, 1))
    J = oracle.sh_real_jacobian(3, r)
    h = 1e-6
    for k in range(3):
        d = np.zeros(3)
        d[k] = h
        fd = (oracle.sh_real(3, r + d) - oracle.sh_real(3, r - d)) / (2 * h)
        assert np.max(np.abs(J[:, :, k] - fd)) <= 1e-7
    assert np.max(np.abs(np.einsum("nbk,nk->nb", J, r))) <= 1e-12
    R = _haar(4)
    JR = oracle.sh_real_jacobian(3, r @ R.T)
    for l in range(4):
        D = oracle.wigner_D_real(l, R)
        s = slice(l * l, (l + 1) ** 2)
        assert np.max(np.abs(JR[:, s, :] - np.einsum("ab,nbk,jk->naj", D, J[:, s, :], R))) <= 1e-11
    P = np.array([[0, 1, 0], [0, 0, 1], [1, 0, 0]], dtype=float)
    nr = np.linalg.norm(r, axis=1)
    u = r / nr[:, None]
    want = np.sqrt(3.0) * (P[None] - np.einsum("ab,nb,nk->nak", P, u, u)) / nr[:, None, None]
    assert np.max(np.abs(J[:, 1:4, :] - want)) <= 1e-13
    # vector-Jacobian product
    gY = rng.normal(size=(40, 16))
    assert np.max(np.abs(oracle.sh_real_vjp(3, r, gY) - np.einsum("nb,nbk->nk", gY, J))) <= 1e-13
