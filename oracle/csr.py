"""Receiver- and sender-grouped edge indices (CSR).

Test infrastructure only (see ``oracle/__init__.py``).

Streaming edges grouped by receiver is what lets receiver-side state replace
scatter atomics ("Sobek: Streaming Equivariant Tensor Product Convolutions",
Abstract; "The GPU Workload That Rewrites Molecular Physics", section "What
Makes MLFF Workloads Structurally Different", on scatter-reduce contention).
The pages fix no tie-break; reading: stable order, ties broken by position.

Returned arrays (all int64 here; the GPU keeps int32):

* ``perm``      -- original edge ids sorted by receiver, stable;
* ``row_ptr``   -- [N+1] receiver offsets into the sorted order;
* ``col``       -- sender of each receiver-sorted edge;
* ``t_perm``    -- receiver-sorted positions regrouped by sender, stable;
* ``t_row_ptr`` -- [N+1] sender offsets into ``t_perm``;
* ``t_col``     -- receiver of each sender-grouped edge.

``launch_order`` orders the nodes of a grouping by descending degree, ties
by ascending node id: the pages name variable degree and hub atoms as what
sets these workloads apart ("The GPU Workload That Rewrites Molecular
Physics", section "What Makes MLFF Workloads Structurally Different"); the
order is a schedule (the largest node first), and the pages fix no tie-break.
"""
import numpy as np


def csr_build(src, dst, n_nodes):
    src = np.asarray(src, dtype=np.int64)
    dst = np.asarray(dst, dtype=np.int64)
    perm = np.argsort(dst, kind="stable")
    row_ptr = np.concatenate([[0], np.cumsum(np.bincount(dst, minlength=n_nodes))])
    col = src[perm]
    t_perm = np.argsort(col, kind="stable")
    t_row_ptr = np.concatenate([[0], np.cumsum(np.bincount(col, minlength=n_nodes))])
    t_col = dst[perm][t_perm]
    return dict(perm=perm, row_ptr=row_ptr, col=col, t_perm=t_perm,
                t_row_ptr=t_row_ptr, t_col=t_col)


def launch_order(ptr):
    """Nodes by descending degree (ptr[i+1] - ptr[i]), ties by node id."""
    deg = np.diff(np.asarray(ptr, dtype=np.int64))
    return np.argsort(-deg, kind="stable")
