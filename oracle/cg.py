"""Clebsch-Gordan coefficients: complex (Racah closed form) and real basis.

Test infrastructure only (see ``oracle/__init__.py``).

The pages name the Clebsch-Gordan tensor product and its sparsity ("FlashTP:
Fused, Sparsity-Aware Tensor Product for MLIPs", Abstract: sparse computation
skips the zeros of this tensor) but never print a coefficient or a phase
convention.  Readings taken here:

* complex CG from Racah's closed form with the Condon-Shortley phase, exact
  rational arithmetic, one square root at the end;
* real basis through the unitary ``U_l`` of :func:`real_basis_matrix`;
* the real tensor of a path is unique up to sign; the sign is fixed so that
  the nonzero entry with the lexicographically smallest (a, b, c) is positive;
* entries with ``|C| <= 1e-12`` are zeros;
* orthonormal in the output index: ``sum_ab C[a,b,c] C[a,b,c'] = delta``,
  with no extra per-path factor.
"""
from fractions import Fraction
from functools import lru_cache
from math import factorial, sqrt

import numpy as np

ZERO_TOL = 1e-12


def _racah_sum(j1, m1, j2, m2, J, M):
    """The alternating sum of Racah's formula, as an exact Fraction."""
    s = Fraction(0)
    kmin = max(0, j2 - J - m1, j1 - J + m2)
    kmax = min(j1 + j2 - J, j1 - m1, j2 + m2)
    for k in range(kmin, kmax + 1):
        den = (factorial(k) * factorial(j1 + j2 - J - k) * factorial(j1 - m1 - k)
               * factorial(j2 + m2 - k) * factorial(J - j2 + m1 + k)
               * factorial(J - j1 - m2 + k))
        s += Fraction((-1) ** k, den)
    return s


@lru_cache(maxsize=None)
def cg_complex(j1, m1, j2, m2, J, M):
    """<j1 m1 j2 m2 | J M> for integer angular momenta (Racah, Condon-Shortley).

    Zero unless M = m1 + m2, |j1 - j2| <= J <= j1 + j2 and every |m| <= j.
    Computed as sign(S) * sqrt(A * S^2) with A and S exact rationals.
    """
    if M != m1 + m2 or J < abs(j1 - j2) or J > j1 + j2:
        return 0.0
    if abs(m1) > j1 or abs(m2) > j2 or abs(M) > J:
        return 0.0
    a = Fraction((2 * J + 1) * factorial(J + j1 - j2) * factorial(J - j1 + j2)
                 * factorial(j1 + j2 - J), factorial(j1 + j2 + J + 1))
    a *= (factorial(J + M) * factorial(J - M) * factorial(j1 - m1)
          * factorial(j1 + m1) * factorial(j2 - m2) * factorial(j2 + m2))
    s = _racah_sum(j1, m1, j2, m2, J, M)
    if s == 0:
        return 0.0
    mag = sqrt(a * s * s)  # Fraction -> float, then one correctly rounded sqrt
    return mag if s > 0 else -mag


def real_basis_matrix(l):
    """Unitary U_l mapping complex (m = -l..l) to real components (rows m = -l..l).

    Reading: the usual real spherical-harmonic combination,
      row m > 0: (-1)^m / sqrt2 at column m,  1/sqrt2 at column -m;
      row m < 0: i / sqrt2 at column m, -i (-1)^|m| / sqrt2 at column |m|;
      row 0:     1 at column 0.
    With Condon-Shortley complex harmonics this gives real harmonics ordered
    (y, z, x) for l = 1.
    """
    n = 2 * l + 1
    U = np.zeros((n, n), dtype=np.complex128)
    r2 = 1.0 / np.sqrt(2.0)
    for m in range(-l, l + 1):
        row = m + l
        if m > 0:
            U[row, m + l] = (-1) ** m * r2
            U[row, -m + l] = r2
        elif m < 0:
            U[row, m + l] = 1j * r2
            U[row, -m + l] = -1j * (-1) ** (-m) * r2
        else:
            U[row, l] = 1.0
    return U


def cg_complex_tensor(l1, l2, l3):
    """Dense complex CG tensor [2l1+1, 2l2+1, 2l3+1] indexed by (m1+l1, m2+l2, m3+l3)."""
    T = np.zeros((2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1))
    for m1 in range(-l1, l1 + 1):
        for m2 in range(-l2, l2 + 1):
            m3 = m1 + m2
            if abs(m3) <= l3:
                T[m1 + l1, m2 + l2, m3 + l3] = cg_complex(l1, m1, l2, m2, l3, m3)
    return T


@lru_cache(maxsize=None)
def _cg_real_cached(l1, l2, l3):
    if l3 < abs(l1 - l2) or l3 > l1 + l2:
        return np.zeros((2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1))
    Cc = cg_complex_tensor(l1, l2, l3)
    U1, U2, U3 = real_basis_matrix(l1), real_basis_matrix(l2), real_basis_matrix(l3)
    # Real inputs t1 = U1 T1, t2 = U2 T2 give T = U^H t; the real output is U3 T3.
    Z = np.einsum("am,bn,co,mno->abc", U1.conj(), U2.conj(), U3, Cc)
    if (l1 + l2 + l3) % 2 == 0:
        T, other = Z.real, Z.imag
    else:
        T, other = Z.imag, Z.real
    if np.max(np.abs(other)) > 1e-14:
        raise AssertionError(f"real CG ({l1},{l2},{l3}) is not purely real/imaginary")
    T = np.where(np.abs(T) > ZERO_TOL, T, 0.0)
    nz = np.argwhere(T != 0.0)  # row-major order = lexicographic (a, b, c)
    if len(nz) and T[tuple(nz[0])] < 0:
        T = -T
    T.setflags(write=False)
    return T


def cg_real(l1, l2, l3):
    """Real-basis CG tensor C[a, b, c] of the path (l1, l2 -> l3), sign-fixed.

    a, b, c index the real components m = -l..l of x (degree l1), Y (degree
    l2) and the output (degree l3).  Returns a read-only float64 array.
    """
    return _cg_real_cached(int(l1), int(l2), int(l3))


def cg_real_nonzeros(l1, l2, l3):
    """List of (a, b, c, value) nonzeros in lexicographic (a, b, c) order."""
    T = cg_real(l1, l2, l3)
    return [(int(a), int(b), int(c), float(T[a, b, c])) for a, b, c in np.argwhere(T != 0.0)]
