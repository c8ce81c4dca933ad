"""Real Wigner-D matrices, used to test equivariance.

Test infrastructure only (see ``oracle/__init__.py``).

Equivariance is the property the pages build on: rotating the atoms must
rotate the predictions ("Accelerating Tensor Products in E(3)-Equivariant
Graph Neural Networks", Abstract).  D^l(R) is defined here by how the real
harmonics transform, ``Y_l(R r) = D^l(R) Y_l(r)``, and found by least squares
over enough random directions; the fit residual is returned so callers can
check it is at rounding level.
"""
import numpy as np

from .sh import sh_real


def wigner_D_real(l, R, n_dirs=None, seed=1234, return_residual=False):
    """D^l(R) with Y_l(R r) = D^l(R) Y_l(r) for every direction r."""
    R = np.asarray(R, dtype=np.float64)
    n = 2 * l + 1
    k = n_dirs or max(4 * n, 16)
    rng = np.random.default_rng(seed)
    r = rng.normal(size=(k, 3))
    sl = slice(l * l, (l + 1) * (l + 1))
    A = sh_real(l, r)[:, sl]
    B = sh_real(l, r @ R.T)[:, sl]
    # B = A D^T
    DT, *_ = np.linalg.lstsq(A, B, rcond=None)
    D = DT.T
    if return_residual:
        return D, float(np.max(np.abs(A @ D.T - B)))
    return D
