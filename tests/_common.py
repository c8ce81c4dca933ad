"""Helpers shared by the tests (no method arithmetic here)."""
import numpy as np


def dims_of(oplan):
    """Sizes a workload needs, read off an oracle plan."""
    return dict(xdim=oplan.xdim, n_paths=oplan.n_paths, U=oplan.U,
                outdim=oplan.outdim, n_out_irreps=len(oplan.out_irreps))


def haar(rng):
    q, r = np.linalg.qr(rng.normal(size=(3, 3)))
    q = q * np.sign(np.diag(r))
    if np.linalg.det(q) < 0:
        q[:, 0] = -q[:, 0]
    return q


def max_rel_block_err(got, ref, offsets_sizes):
    """max over blocks of max|got-ref| / max|ref| (columns grouped by block)."""
    worst = 0.0
    for off, size in offsets_sizes:
        r = ref[..., off:off + size]
        g = got[..., off:off + size]
        scale = float(np.max(np.abs(r))) if r.size else 0.0
        err = float(np.max(np.abs(g - r))) if r.size else 0.0
        worst = max(worst, err / scale if scale > 0 else err)
    return worst
