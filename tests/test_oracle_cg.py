"""Pins for the oracle's Clebsch-Gordan coefficients and path tables.

Each check compares the oracle with something that is not the oracle: sympy's
exact CG routine, printed textbook values, orthogonality and symmetry
relations of the coupling coefficients, closed forms of the real tensors, and
rotation equivariance with Wigner-D matrices built from the harmonics.
"""
import os
from math import sqrt  # noqa: F401  (used by eval of the golden file)

import numpy as np
import pytest
from sympy.physics.wigner import clebsch_gordan as sympy_cg

import oracle
from oracle.cg import cg_complex_tensor

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "cg_textbook.txt")


def _triples(lmax):
    for l1 in range(lmax + 1):
        for l2 in range(lmax + 1):
            for l3 in range(abs(l1 - l2), min(l1 + l2, lmax) + 1):
                yield l1, l2, l3


def test_complex_cg_matches_sympy_exact():
    worst = 0.0
    for l1, l2, J in _triples(4):
        for m1 in range(-l1, l1 + 1):
            for m2 in range(-l2, l2 + 1):
                M = m1 + m2
                if abs(M) > J:
                    continue
                ref = float(sympy_cg(l1, l2, J, m1, m2, M))
                worst = max(worst, abs(oracle.cg_complex(l1, m1, l2, m2, J, M) - ref))
    assert worst <= 1e-15


def test_complex_cg_textbook_values():
    n = 0
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        f = line.split()
        j1, m1, j2, m2, J, M = map(int, f[:6])
        want = eval(f[6])
        assert abs(oracle.cg_complex(j1, m1, j2, m2, J, M) - want) <= 1e-15, line
        n += 1
    assert n >= 20


@pytest.mark.parametrize("j", [0, 1, 2, 3, 4])
def test_complex_cg_closed_forms(j):
    # <j m j -m | 0 0> = (-1)^(j-m) / sqrt(2j+1)
    for m in range(-j, j + 1):
        want = (-1) ** (j - m) / np.sqrt(2 * j + 1)
        assert abs(oracle.cg_complex(j, m, j, -m, 0, 0) - want) <= 1e-15
    # stretched state <l1 l1 l2 l2 | l1+l2, l1+l2> = 1
    for l2 in range(0, 4):
        assert abs(oracle.cg_complex(j, j, l2, l2, j + l2, j + l2) - 1.0) <= 1e-15


def test_complex_cg_orthogonality_and_symmetry():
    for l1 in range(4):
        for l2 in range(4):
            Js = range(abs(l1 - l2), l1 + l2 + 1)
            # Full unitary matrix (m1, m2) x (J, M).
            rows = [(m1, m2) for m1 in range(-l1, l1 + 1) for m2 in range(-l2, l2 + 1)]
            cols = [(J, M) for J in Js for M in range(-J, J + 1)]
            A = np.array([[oracle.cg_complex(l1, m1, l2, m2, J, M) for J, M in cols]
                          for m1, m2 in rows])
            assert np.max(np.abs(A.T @ A - np.eye(len(cols)))) <= 1e-14
            assert np.max(np.abs(A @ A.T - np.eye(len(rows)))) <= 1e-14
            # swap symmetry <l2 m2 l1 m1|J M> = (-1)^(l1+l2-J) <l1 m1 l2 m2|J M>
            for J in Js:
                for m1 in range(-l1, l1 + 1):
                    for m2 in range(-l2, l2 + 1):
                        a = oracle.cg_complex(l1, m1, l2, m2, J, m1 + m2)
                        b = oracle.cg_complex(l2, m2, l1, m1, J, m1 + m2)
                        assert abs(b - (-1) ** (l1 + l2 - J) * a) <= 1e-15


def test_real_basis_is_unitary():
    for l in range(6):
        U = oracle.real_basis_matrix(l)
        assert np.max(np.abs(U @ U.conj().T - np.eye(2 * l + 1))) <= 1e-15


def test_real_cg_orthonormal_and_complete():
    for l1 in range(4):
        for l2 in range(4):
            stack = []
            for l3 in range(abs(l1 - l2), l1 + l2 + 1):
                C = oracle.cg_real(l1, l2, l3)
                n3 = 2 * l3 + 1
                G = np.einsum("abc,abd->cd", C, C)
                assert np.max(np.abs(G - np.eye(n3))) <= 1e-14
                stack.append(C.reshape(-1, n3))
            # completeness: sum_{l3,c} C[a,b,c] C[a',b',c] = delta delta
            S = np.concatenate(stack, axis=1)
            assert np.max(np.abs(S @ S.T - np.eye(S.shape[0]))) <= 1e-14


def test_real_cg_from_sympy_route():
    """Real tensors rebuilt from sympy's CG agree up to the stated sign rule."""
    for l1, l2, l3 in _triples(3):
        Cc = np.zeros((2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1))
        for m1 in range(-l1, l1 + 1):
            for m2 in range(-l2, l2 + 1):
                if abs(m1 + m2) <= l3:
                    Cc[m1 + l1, m2 + l2, m1 + m2 + l3] = float(
                        sympy_cg(l1, l2, l3, m1, m2, m1 + m2))
        U1, U2, U3 = (oracle.real_basis_matrix(l) for l in (l1, l2, l3))
        Z = np.einsum("am,bn,co,mno->abc", U1.conj(), U2.conj(), U3, Cc)
        T = Z.real if (l1 + l2 + l3) % 2 == 0 else Z.imag
        T = np.where(np.abs(T) > 1e-12, T, 0.0)
        first = tuple(np.argwhere(T != 0)[0])
        if T[first] < 0:
            T = -T
        assert np.max(np.abs(T - oracle.cg_real(l1, l2, l3))) <= 1e-15


def test_real_cg_closed_forms():
    for l in range(5):
        n = 2 * l + 1
        I = np.eye(n)
        # (0, l, l) and (l, 0, l): identity; (l, l, 0): delta_ab / sqrt(2l+1)
        assert np.max(np.abs(oracle.cg_real(0, l, l)[0] - I)) <= 1e-15
        assert np.max(np.abs(oracle.cg_real(l, 0, l)[:, 0, :] - I)) <= 1e-15
        assert np.max(np.abs(oracle.cg_real(l, l, 0)[:, :, 0] - I / np.sqrt(n))) <= 1e-15
    # (1, 1, 1): cross product / sqrt2 in the (y, z, x) component order
    C = oracle.cg_real(1, 1, 1)
    rng = np.random.default_rng(0)
    for _ in range(5):
        a, b = rng.normal(size=3), rng.normal(size=3)   # Cartesian (x, y, z)
        P = [1, 2, 0]                                    # (x,y,z) -> (y,z,x)
        got = np.einsum("abc,a,b->c", C, a[P], b[P])
        want = np.cross(a, b)[P] / np.sqrt(2.0)
        assert np.max(np.abs(got - want)) <= 1e-15


def _haar(rng):
    q, r = np.linalg.qr(rng.normal(size=(3, 3)))
    q = q * np.sign(np.diag(r))
    if np.linalg.det(q) < 0:
        q[:, 0] = -q[:, 0]
    return q


def test_real_cg_equivariance():
    rng = np.random.default_rng(7)
    R = _haar(rng)
    D = {l: oracle.wigner_D_real(l, R) for l in range(5)}
    for l1, l2, l3 in _triples(4):
        C = oracle.cg_real(l1, l2, l3)
        lhs = np.einsum("abc,ai,bj->ijc", C, D[l1], D[l2])
        rhs = np.einsum("ck,ijk->ijc", D[l3], C)
        assert np.max(np.abs(lhs - rhs)) <= 1e-13


def test_parity_selection_is_respected():
    # A path whose output parity differs from (-1)^(l1+l2) would break
    # inversion symmetry; the complex tensor vanishes only by the triangle rule,
    # so every allowed path must carry nonzeros.
    for l1, l2, l3 in _triples(4):
        assert np.count_nonzero(oracle.cg_real(l1, l2, l3)) > 0


# Nonzero counts of the real tensors; the same counts come out of sympy's
# exact coefficients through the route of test_real_cg_from_sympy_route.
def _nnz_via_sympy(l1, l2, l3):
    Cc = np.zeros((2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1))
    for m1 in range(-l1, l1 + 1):
        for m2 in range(-l2, l2 + 1):
            if abs(m1 + m2) <= l3:
                Cc[m1 + l1, m2 + l2, m1 + m2 + l3] = float(sympy_cg(l1, l2, l3, m1, m2, m1 + m2))
    U1, U2, U3 = (oracle.real_basis_matrix(l) for l in (l1, l2, l3))
    Z = np.einsum("am,bn,co,mno->abc", U1.conj(), U2.conj(), U3, Cc)
    return int(np.count_nonzero(np.abs(Z) > 1e-12))


@pytest.mark.parametrize("irreps,lsh,lout,P,nnz,xdim,outdim,outs", [
    ("8x0e+8x1o", 2, 2, 9, 59, 32, 136, "8x0e+8x1e+8x1o+8x2e+8x2o"),
    ("32x0e+32x1o+32x2e", 2, 2, 15, 137, 288, 544, "32x0e+32x1e+32x1o+32x2e+32x2o"),
    ("64x0e+64x1o+64x2e+64x3o", 3, 3, 34, 611, 1024, 1984,
     "64x0e+64x1e+64x1o+64x2e+64x2o+64x3e+64x3o"),
])
def test_plan_tables(irreps, lsh, lout, P, nnz, xdim, outdim, outs):
    plan = oracle.build_plan(irreps, lsh, lout)
    assert plan.n_paths == P
    assert plan.nnz() == nnz
    assert plan.xdim == xdim and plan.outdim == outdim
    assert plan.out_irreps_str() == outs
    assert sum(_nnz_via_sympy(l1, l2, l3) for _, l1, l2, l3, _ in plan.paths) == nnz
    for (_, l1, l2, l3, k), C in zip(plan.paths, plan.cg):
        assert plan.out_irreps[k] == (l3, (-1) ** (l1 + l2))
        assert C.shape == (2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1)


def test_parse_errors():
    for bad in ["", "8x0e+", "8x0q", "x0e", "0x0e", "8x1e", "8x0e+4x1o"]:
        with pytest.raises(ValueError):
            oracle.build_plan(bad, 2, 2)
