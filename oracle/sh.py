"""Real spherical harmonics of edge directions.

Test infrastructure only (see ``oracle/__init__.py``).

The pages say the convolution couples node features with spherical harmonics
of the edge direction ("The GPU Workload That Rewrites Molecular Physics",
section "What Makes MLFF Workloads Structurally Different": equivariant
feature transforms over spherical harmonics and CG products) without fixing a
basis.  Reading: component normalisation, ``Y_l = sqrt(4 pi) U_l Y_l^complex``
with Condon-Shortley complex harmonics and ``U_l`` from
:func:`oracle.cg.real_basis_matrix`, so ``sum_m Y_lm^2 = 2l+1`` and
``Y_1 = sqrt3 (y, z, x)`` for a unit vector.
"""
from math import factorial

import numpy as np

from .cg import real_basis_matrix


def _assoc_legendre(l, m, x):
    """P_l^m(x) for 0 <= m <= l with the Condon-Shortley phase (3-term recurrence)."""
    x = np.asarray(x, dtype=np.float64)
    pmm = np.ones_like(x)
    if m > 0:
        s = np.sqrt(np.clip(1.0 - x * x, 0.0, None))
        dfact = 1.0
        for k in range(1, 2 * m, 2):
            dfact *= k
        pmm = (-1) ** m * dfact * s ** m
    if l == m:
        return pmm
    pm1 = x * (2 * m + 1) * pmm
    if l == m + 1:
        return pm1
    p_prev, p_cur = pmm, pm1
    for ll in range(m + 2, l + 1):
        p_next = ((2 * ll - 1) * x * p_cur - (ll + m - 1) * p_prev) / (ll - m)
        p_prev, p_cur = p_cur, p_next
    return p_cur


def sh_complex(l, r):
    """Complex orthonormal Y_l^m(r_hat) for m = -l..l, shape [n, 2l+1]."""
    r = np.asarray(r, dtype=np.float64).reshape(-1, 3)
    n = np.linalg.norm(r, axis=1)
    z = r[:, 2] / n
    phi = np.arctan2(r[:, 1], r[:, 0])
    out = np.zeros((r.shape[0], 2 * l + 1), dtype=np.complex128)
    for m in range(0, l + 1):
        norm = np.sqrt((2 * l + 1) / (4 * np.pi) * factorial(l - m) / factorial(l + m))
        ylm = norm * _assoc_legendre(l, m, z) * np.exp(1j * m * phi)
        out[:, l + m] = ylm
        if m > 0:
            out[:, l - m] = (-1) ** m * np.conj(ylm)
    return out


def sh_real(lmax, r):
    """Real component-normalised harmonics of the directions of r, [n, (lmax+1)^2].

    Columns are l-blocks (l = 0..lmax), each with m = -l..l.  The length of r
    does not matter; a zero vector is not a direction and is rejected.
    """
    r = np.asarray(r, dtype=np.float64).reshape(-1, 3)
    if np.any(np.linalg.norm(r, axis=1) == 0.0):
        raise ValueError("zero-length edge vector has no direction")
    blocks = []
    for l in range(lmax + 1):
        Z = np.sqrt(4 * np.pi) * sh_complex(l, r) @ real_basis_matrix(l).T
        if np.max(np.abs(Z.imag), initial=0.0) > 1e-12:
            raise AssertionError("real harmonics came out complex")
        blocks.append(Z.real)
    return np.concatenate(blocks, axis=1)


# ---------------------------------------------------------------------------
# Gradient with respect to the edge vector (forces flow through Y).
#
# R_lm(r) = |r|^l Y_lm(r_hat) is a homogeneous polynomial of degree l (a solid
# harmonic).  Its monomial coefficients are obtained here by interpolating
# sh_real at more points than there are monomials of degree l (an exact
# interpolation of a polynomial of known degree, up to rounding); then
#   dY/dr = grad R(r) / |r|^l - l R(r) r / |r|^(l+2),
# which is zero along r, as it must be for a function of the direction only.
# ---------------------------------------------------------------------------

def _monomial_exponents(l):
    return [(a, b, l - a - b) for a in range(l, -1, -1) for b in range(l - a, -1, -1)]


def _monomials(exps, r):
    x, y, z = r[:, 0:1], r[:, 1:2], r[:, 2:3]
    return np.concatenate([x ** a * y ** b * z ** c for a, b, c in exps], axis=1)


_SOLID = {}


def solid_harmonic_coefficients(l):
    """[2l+1, n_monomials] coefficients of R_lm in the monomials of degree l."""
    if l not in _SOLID:
        exps = _monomial_exponents(l)
        rng = np.random.default_rng(12345)
        u = rng.normal(size=(4 * len(exps) + 8, 3))
        u /= np.linalg.norm(u, axis=1, keepdims=True)
        Y = sh_real(l, u)[:, l * l:]                 # on the unit sphere R = Y
        M = _monomials(exps, u)
        C, *_ = np.linalg.lstsq(M, Y, rcond=None)
        if np.max(np.abs(M @ C - Y)) > 1e-12:
            raise AssertionError("solid harmonic is not a polynomial of degree l")
        _SOLID[l] = (exps, C.T.copy())
    return _SOLID[l]


def sh_real_jacobian(lmax, r):
    """dY/dr, shape [n, (lmax+1)^2, 3], for the harmonics of sh_real."""
    r = np.asarray(r, dtype=np.float64).reshape(-1, 3)
    nr = np.linalg.norm(r, axis=1)
    if np.any(nr == 0.0):
        raise ValueError("zero-length edge vector has no direction")
    J = np.zeros((r.shape[0], (lmax + 1) ** 2, 3))
    for l in range(1, lmax + 1):
        exps, C = solid_harmonic_coefficients(l)
        R = _monomials(exps, r) @ C.T                                  # [n, 2l+1]
        grad = np.zeros((r.shape[0], 2 * l + 1, 3))
        for axis in range(3):
            dexps, scale = [], []
            for e in exps:
                k = e[axis]
                d = list(e)
                d[axis] = max(k - 1, 0)
                dexps.append(tuple(d))
                scale.append(float(k))
            dm = _monomials(dexps, r) * np.array(scale)[None, :]
            grad[:, :, axis] = dm @ C.T
        s = nr[:, None, None]
        J[:, l * l:(l + 1) ** 2, :] = grad / s ** l - l * R[:, :, None] * r[:, None, :] / s ** (l + 2)
    return J


def sh_real_vjp(lmax, r, grad_Y):
    """grad_r[e] = sum_b grad_Y[e, b] dY_b/dr[e]."""
    return np.einsum("nb,nbk->nk", np.asarray(grad_Y, dtype=np.float64), sh_real_jacobian(lmax, r))
