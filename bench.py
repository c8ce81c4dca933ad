"""Throughput of the fused tensor-product convolution on one MI355X.

A step is one pass of the hot path over one batch: the forward kernel and the
backward (gradients with respect to x, w and Y) of one layer.  The default
run measures the 1,536-atom / 46,080-edge workload (32x0e+32x1o+32x2e,
harmonics to l = 2, every path with l3 <= 2, channel-wise weights) as the
headline ``value`` and, in ``configs``, the other four workloads: the 32-atom
tiny graph, the 4,096-atom lmax-3 forward, the 32,768-atom power-law (Zipf)
graph at lmax 3, and the 100,000-atom / 3,000,000-edge streaming layer with
on-chip radial weights and the channel mix.  ``--config NAME`` measures one
workload alone (used for profiler runs).  The graph preparation (CSR build
and launch order) is timed separately: it runs once per neighbour list, not
per layer.  Every pass walks its nodes in the launch order (largest degree
first); the direct-weight and radial lines also time the same step in node
order, and the lmax-2 direct-weight lines the step with the edge rows in
the sender grouping.

Timing, every figure cold (nothing of the step's edge-sized inputs in L2 or
the 256 MB Infinity Cache):
  * steps: W untimed warm-up steps, then K timed steps back to back in one
    bracket of HIP events on the stream the kernels run on (torch's current
    stream), after a 1 GiB read of an unrelated buffer; the steps rotate
    over enough full copies of everything a step touches (graph, features,
    weights, harmonics, gradients, outputs) that a copy is reused only after
    at least 1 GiB of other data, so no step finds its inputs in L2 or the
    Infinity Cache.  Where that many copies would not reach 1 GiB (the
    32-atom graph) and for the radial, fully connected and Gaunt lines, each
    step follows the flush in its own event bracket; the direct-weight lines
    report that isolated step beside the stream (ms_per_step_isolated);
  * kernels: back-to-back launches that rotate through enough copies of the
    edge-sized inputs and outputs that a copy is reused only after at least
    1 GiB of other edge data has been touched (one copy where a single
    launch already moves more than that); the per-launch duration is the
    event-timed batch divided by the launch count.  ``--warm`` also times
    steps without the flush.

Output: one JSON line.  ``value`` is edges per second of forward + backward
on the 1,536-atom workload; ``roofline`` reports its slowest kernel against
the 8 TB/s HBM peak with that kernel's algorithmic bytes, ``step_roofline``
the whole step against the bytes it must move (each array once per pass);
``valu_flop_util`` the fp32 vector flops of the CG arithmetic per second
against 78.6 TFLOP/s; ``cpu_baseline`` the float64 oracle on this host's
cores (a process pool over edge chunks) on the same workload.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TP-conv edges/sec (fwd, fwd+bwd) fp32 at 1 GPU; % of MI355X HBM roofline"
HBM_PEAK_GBS = 8000.0
FP32_MFMA_PEAK_TFLOPS = 157.3
FP32_VALU_PEAK_TFLOPS = 78.6      # non-packed fp32 FMA: 256 CUs x 4 SIMDs x 16 lanes x 2 x 2.4 GHz
COLD_BYTES = 1 << 30              # edge data touched between two uses of one copy
HOST_POOL_CAP = 16                # host cores of one GPU's share on the box
WORKLOADS = {
    "mid": ("32x0e+32x1o+32x2e", 2, 2,
            "1536 atoms, 46080 directed edges (30 distinct random senders each), "
            "32x0e+32x1o+32x2e, real SH lmax 2, all paths l3<=2 (15), uvu weights, fwd+bwd"),
    "tiny": ("8x0e+8x1o", 2, 2, "32 atoms in an 8 A periodic cube, cutoff 4 A, 8x0e+8x1o, fwd+bwd"),
    "lmax3": ("64x0e+64x1o+64x2e+64x3o", 3, 3,
              "4096 atoms, degree U{5..30}, 64x(0e+1o+2e+3o), SH lmax 3, 34 paths, fwd"),
    "zipf": ("64x0e+64x1o+64x2e+64x3o", 3, 3,
             "32768 atoms, Zipf(1.5) receiver degrees capped at 256, 64x(0e+1o+2e+3o), "
             "SH lmax 3, 34 paths, fwd+bwd"),
}
RADIAL_WORKLOADS = {
    "stream": ("128x0e+128x1o+128x2e", 2, 2, (8, 64, 5.0),
               "100000 atoms, 3000000 directed edges (30 distinct random senders each, length "
               "U[0.8,5] A), 128x0e+128x1o+128x2e, real SH lmax 2, all paths l3<=2 (15), edge "
               "weights from a radial MLP (8 Bessel -> 64 SiLU -> 15x128) computed on chip, "
               "128x128 uvw mix per output irrep, fwd+bwd"),
    "lmax3_radial": ("64x0e+64x1o+64x2e+64x3o", 3, 3, (8, 64, 5.0),
                     "4096 atoms, degree U{5..30} (length U[0.8,5] A), 64x(0e+1o+2e+3o), SH lmax 3, 34 "
                     "paths, edge weights from a radial MLP (8 Bessel -> 64 SiLU -> 34x64) computed on "
                     "chip, 64x64 uvw mix per output irrep, fwd+bwd"),
}
FC_WORKLOADS = {
    "fc": ("32x0e+32x1o+32x2e", 2, 2, 8,
           "1536 atoms, 46080 directed edges (the mid graph), 32x0e+32x1o+32x2e, real SH lmax 2, "
           "15 paths, fully connected per-edge weights W_e = sum_h R_e[h] Theta[h] (8 radial "
           "features, 32x32 per path) by reassociation into receiver state, fwd+bwd"),
}
GAUNT_WORKLOADS = {
    "gaunt": ("32x0e+32x1o+32x2e", 2, 2,
              "1536 atoms, 46080 directed edges (the mid graph), 32x0e+32x1o+32x2e, real SH lmax 2, "
              "Gaunt product (even couplings, outputs 0e+1o+2e) evaluated on a 32-point spherical "
              "grid, filter weights per edge, degree and channel, fwd+bwd"),
}
DEFAULT_CONFIGS = ("tiny", "lmax3", "zipf", "stream", "lmax3_radial")
GAUNT_SOURCES = ("gaunt.hip",)
PROFILE_SUMMARY = os.path.join(ROOT, "profiles", "hbm_traffic_{}.txt")
KERNEL_SOURCES = ("conv_kernels.hpp", "sig.hpp", "cg_table.hpp")
RADIAL_SOURCES = {      # per radial workload: the sources its kernels are built from
    "stream": ("radial_kernels.hpp", "radial_dbl_kernels.hpp", "radial_launch.hpp", "radial_l012_s2.hip",
               "uvw.hip", "conv_kernels.hpp", "sig.hpp", "cg_table.hpp"),
    "lmax3_radial": ("radial_kernels.hpp", "radial_launch.hpp", "radial_l0123_s3.hip", "uvw.hip",
                     "conv_kernels.hpp", "sig.hpp", "cg_table.hpp"),
}
FC_SOURCES = ("fc_kernels.hip", "radial_kernels.hpp", "conv_kernels.hpp", "sig.hpp", "cg_table.hpp")


def kernel_source_hash(sources=KERNEL_SOURCES):
    h = hashlib.sha256()
    d = os.path.join(ROOT, "tensor_product_convolution_amd", "csrc")
    for f in sources:
        h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def one_pass_backward(lmax_sh):
    """tp_conv_backward forms every gradient in one sender-grouped launch for the
    lmax-2 signatures, and in a receiver pass plus a sender pass otherwise."""
    return lmax_sh <= 2


def algorithmic_bytes(N, E, P, U, ysh, xdim, outdim):
    """Bytes each kernel must move at least once (node arrays once, edge streams once)."""
    node = 4 * N * (xdim + outdim + 1)        # x, out (or grad_out / grad_x), row pointers
    return {
        "fwd": E * (4 * P * U + 4 * ysh + 4) + node,          # w, Y, col in; out
        "bwd_recv": E * (8 * P * U + 8 * ysh + 4) + node,     # w, Y, col in; grad_w, grad_Y out
        "bwd_send": E * (4 * P * U + 4 * ysh + 8) + node,     # w, Y, t_perm, t_col in; grad_x out
        # one-pass backward: w, Y, t_perm, t_col in, grad_w, grad_Y out; x, grad_out,
        # t_row_ptr in, grad_x out
        "bwd": E * (8 * P * U + 8 * ysh + 8) + 4 * N * (2 * xdim + outdim + 1),
        # sender-grouped layout: the forward also reads e_pos, the backward no t_perm
        "fwd_sg": E * (4 * P * U + 4 * ysh + 8) + node,
        "bwd_sg": E * (8 * P * U + 8 * ysh + 4) + 4 * N * (2 * xdim + outdim + 1),
        # compulsory bytes of the whole step: each array once
        "step": E * (8 * P * U + 8 * ysh + 4) + 4 * N * (2 * xdim + 2 * outdim + 1),
        # second-order backward, each array once: w, gg_w, Y, gg_Y, col, t_perm,
        # t_col in, d_w and d_Y out; x, gg_x, grad_out and both row pointers in,
        # d_x and d_grad_out out
        "double_bwd": E * (12 * P * U + 12 * ysh + 12) + 4 * N * (3 * xdim + 2 * outdim + 2),
    }


def algorithmic_bytes_geom(N, E, P, U, xdim, outdim):
    """The same counts for the edge-vector form: r [E, 3] (12 B) in place of Y,
    grad_r (12 B) in place of grad_Y."""
    return {
        "fwd_r": E * (4 * P * U + 12 + 4) + 4 * N * (xdim + outdim + 1),     # w, r, col; x, out
        # w, r, t_perm, t_col in, grad_w, grad_r out; x, grad_out, t_row_ptr in, grad_x out
        "bwd_r": E * (8 * P * U + 24 + 8) + 4 * N * (2 * xdim + outdim + 1),
    }


def step_bytes(ab, fwd_only):
    """Bytes a forward (+ backward) pass must move, each pass touching its arrays
    once: the forward's and the one-pass backward's algorithmic bytes."""
    return ab["fwd"] if fwd_only else ab["fwd"] + ab["bwd"]


def cg_counts(paths, pabc, val):
    """Operation counts of the CG arithmetic per edge and channel, from the
    plan's path list ((l1, l2, l3, k) per path) and nonzeros ((p, a, b, c), C):
    nnz; the coupled (a, b) pairs of each (l1, l2) group (the shared products
    x_a Y_b and the grad_x folds); sum over paths of 2l2+1 and of 2l3+1; and
    the distinct nontrivial magnitudes |C| per output component (the one-pass
    backward's scaled upstream-gradient values)."""
    ab, gc = set(), set()
    for (p, a, b, c), v in zip(pabc, val):
        l1, l2, l3, k = paths[p]
        ab.add((l1, l2, int(a), int(b)))
        m = float(np.float32(abs(v)))
        if m != 1.0:
            gc.add((k, int(c), m))
    return {"nnz": len(val), "ab": len(ab), "d2": sum(2 * q[1] + 1 for q in paths),
            "d3": sum(2 * q[2] + 1 for q in paths), "gc": len(gc)}


def cg_flops(cnt):
    """fp32 vector flops per edge and channel (multiply 1, fused multiply-add 2)
    of the CG arithmetic in the forms the kernels evaluate:
      fwd       products x_a Y_b, one FMA per nonzero, one FMA per (path, c) with w;
      bwd       (one pass) scaled gradients, two FMAs per nonzero (Z and V forms),
                grad_w and grad_Y folds over (path, b), grad_x folds over (a, b);
      bwd_recv  multiply + FMA per nonzero (Z form), grad_w and grad_Y folds;
      bwd_send  w g products, one FMA per nonzero, grad_x folds."""
    fl = {"fwd": cnt["ab"] + 2 * cnt["nnz"] + 2 * cnt["d3"],
          "bwd": cnt["gc"] + 4 * cnt["nnz"] + 4 * cnt["d2"] + 2 * cnt["ab"],
          "bwd_recv": 3 * cnt["nnz"] + 4 * cnt["d2"],
          "bwd_send": cnt["d3"] + 2 * cnt["nnz"] + 2 * cnt["ab"]}
    fl["fwd_sg"], fl["bwd_sg"] = fl["fwd"], fl["bwd"]     # same arithmetic in the sender layout
    return fl


def radial_flops(E, P, U, NH):
    """MFMA flops per launch: each pass forms [E x NH] x [NH x P*U] products."""
    mlp = 2.0 * NH * P * U * E
    # second-order backward: w and its tangent v (forward tangent and sender
    # passes), w, v, dh and dt (receiver pass), h^T dw and t^T dv (d_W2)
    return {"fwd": mlp, "bwd_recv": 2 * mlp, "bwd_w2": mlp, "bwd_send": mlp, "double_bwd": 10 * mlp}


def read_traffic(config, sources=KERNEL_SOURCES):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None."""
    path = PROFILE_SUMMARY.format(config)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        line = line.strip()
        if line.startswith("#") or "=" not in line:
            continue
        k, v = line.split("=", 1)
        vals[k.strip()] = v.strip()
    if vals.get("kernel_source_hash") != kernel_source_hash(sources):
        return None          # kernels changed since the counters were taken
    out = {}
    for k, v in vals.items():
        if k.startswith("traffic_bytes."):
            out[k.split(".", 1)[1]] = float(v)
    return out or None


def read_profile_value(config, key, sources):
    """one value of the committed counter summary (None if absent or stale)"""
    path = PROFILE_SUMMARY.format(config)
    if not os.path.exists(path):
        return None
    vals = dict(l.split("=", 1) for l in open(path) if "=" in l and not l.startswith("#"))
    vals = {k.strip(): v.strip() for k, v in vals.items()}
    if vals.get("kernel_source_hash") != kernel_source_hash(sources):
        return None
    return float(vals[key]) if key in vals else None


def copies_for_cold(bytes_per_copy):
    """Copies of the edge-sized arrays so that one is reused only after
    COLD_BYTES of other edge data (at most 16)."""
    return int(min(16, max(1, math.ceil(COLD_BYTES / max(bytes_per_copy, 1)))))


# ---------------------------------------------------------------------------
# CPU baseline: the float64 oracle over a process pool


def host_workers():
    return max(1, min(HOST_POOL_CAP, len(os.sched_getaffinity(0))))


_POOL_STATE = {}


def _pool_init(plan_args):
    try:
        from threadpoolctl import threadpool_limits
        _POOL_STATE["limits"] = threadpool_limits(1)
    except Exception:
        pass
    import oracle
    _POOL_STATE["op"] = oracle.build_plan(*plan_args)


def _oracle_direct_chunk(task):
    """harmonics + forward (+ backward) of one chunk of edges (whole receivers)"""
    import oracle
    op = _POOL_STATE["op"]
    src, dst, n, x, r, w, g = task
    Y = oracle.sh_real(op.lmax_sh, r)
    res = [oracle.tp_conv_fwd(op, src, dst, n, x, Y, w)]
    if g is not None:
        res.extend(oracle.tp_conv_bwd(op, src, dst, n, x, Y, w, g))
    return res


def _oracle_radial_chunk(task):
    import oracle
    op = _POOL_STATE["op"]
    src, dst, n, x, r, rl, W1, W2, Wm, g, nb, rc = task
    Y = oracle.sh_real(op.lmax_sh, r)
    out = oracle.tp_conv_radial_fwd(op, src, dst, n, x, Y, rl, W1, W2, Wm, nb, rc)
    return [out, oracle.tp_conv_radial_bwd(op, src, dst, n, x, Y, rl, W1, W2, Wm, g, nb, rc)]


def _receiver_sample(src, dst, max_edges):
    """Edges into the first receivers (whole receivers, at most max_edges)."""
    order = np.argsort(dst, kind="stable")
    if len(order) <= max_edges:
        return np.arange(len(src)), f"the whole workload ({len(src)} edges)"
    keep = order[:max_edges]
    last = dst[keep[-1]]
    keep = keep[dst[keep] != last]
    return np.sort(keep), f"edges into the first receivers ({len(keep)} of {len(src)} edges)"


def _chunks_by_receiver(dst, n_chunks):
    """Split edge indices into chunks of whole receivers, balanced by edge count."""
    order = np.argsort(dst, kind="stable")
    bounds = np.linspace(0, len(order), n_chunks + 1).astype(np.int64)
    cuts = [0]
    for b in bounds[1:-1]:
        while b < len(order) and b > 0 and dst[order[b]] == dst[order[b - 1]]:
            b += 1
        cuts.append(max(b, cuts[-1]))
    cuts.append(len(order))
    return [order[cuts[t]:cuts[t + 1]] for t in range(n_chunks) if cuts[t + 1] > cuts[t]]


def _local(src, dst, chunk, *node_arrays):
    """The chunk's edges renumbered over the nodes they touch, with those nodes' rows."""
    nodes = np.unique(np.concatenate([src[chunk], dst[chunk]]))
    ls, ld = np.searchsorted(nodes, src[chunk]), np.searchsorted(nodes, dst[chunk])
    return nodes, ls, ld, [None if a is None else a[nodes] for a in node_arrays]


def _block_err(got, ref, blocks):
    """max over column blocks of max|got - ref| / max|ref| of the block"""
    worst = 0.0
    for sl in blocks:
        r, g = ref[:, sl], got[:, sl]
        if r.size == 0:
            continue
        scale = float(np.max(np.abs(r)))
        err = float(np.max(np.abs(g - r)))
        worst = max(worst, err / scale if scale > 0 else err)
    return worst


def _cg_blocks(plan_args):
    """column blocks of a CG plan's arrays: output and input irreps, harmonic
    degrees, weight paths"""
    import oracle
    op = oracle.build_plan(*plan_args)
    U = op.U
    return {
        "out": [slice(o, o + U * (2 * l + 1)) for (l, _), o in zip(op.out_irreps, op.out_offsets)],
        "x": [slice(o, o + U * (2 * l + 1)) for (_, l, _), o in zip(op.irreps_in, op.in_offsets)],
        "Y": [slice(l * l, (l + 1) ** 2) for l in range(op.lmax_sh + 1)],
        "w": [slice(p * U, (p + 1) * U) for p in range(op.n_paths)],
        "all": [slice(None)],
    }


def _parity(plan_args, e, recv_rows, checks, what, blocks=None):
    """Parity of the timed run against the oracle on the CPU-baseline sample:
    checks is a list of (name, got, ref, kind), kind a key of the column blocks
    (those of the CG plan unless given; rows already aligned); the
    block-relative error of each and their max."""
    blocks = blocks or _cg_blocks(plan_args)
    errs = {}
    for name, got, ref, kind in checks:
        got = np.asarray(got, dtype=np.float64).reshape(len(got), -1)
        ref = np.asarray(ref, dtype=np.float64).reshape(len(ref), -1)
        errs[name] = _block_err(got, ref, blocks[kind])
    return {"max_rel_err": max(errs.values()), "per_output": errs, "tol": 1e-4,
            "sample": f"{what}: rows of {recv_rows} receivers with all their edges, and those edges",
            "note": "largest max|gpu - oracle| / max|oracle| over the irrep, path and degree blocks; "
                    "the GPU values are those of the timed step"}


def pooled_oracle_direct(plan_args, src, dst, n, x, r, w, g, workers):
    """The oracle's harmonics + forward (+ backward when g is given) for the edges
    (src, dst), split by receiver over a process pool (each task carries only
    the rows of the nodes its edges touch); returns (out, grad_x, grad_Y,
    grad_w) in the given edge order (grads None without g) and the wall time of
    the pooled evaluation (preparing and distributing the tasks and collecting
    the results included; the pool's start-up and plan building excluded)."""
    import multiprocessing as mp
    ctx = mp.get_context("fork")
    with ctx.Pool(workers, initializer=_pool_init, initargs=(plan_args,)) as pool:
        pool.map(_oracle_direct_chunk, [(src[:0], dst[:0], 1, x[:1], r[:0], w[:0],
                                         None if g is None else g[:1])] * workers)   # warm
        t0 = time.perf_counter()
        chunks = _chunks_by_receiver(dst, workers)
        tasks, maps = [], []
        for c in chunks:
            nodes, ls, ld, (xc, gc) = _local(src, dst, c, x, g)
            tasks.append((ls, ld, len(nodes), xc, r[c], w[c], gc))
            maps.append(nodes)
        parts = pool.map(_oracle_direct_chunk, tasks)
        out = np.zeros((n,) + parts[0][0].shape[1:])
        for nodes, p in zip(maps, parts):
            out[nodes] += p[0]
        grads = (None, None, None)
        if g is not None:
            gx = np.zeros((n,) + parts[0][1].shape[1:])
            gY = np.zeros((len(src),) + parts[0][2].shape[1:])
            gw = np.zeros((len(src),) + parts[0][3].shape[1:])
            for c, nodes, p in zip(chunks, maps, parts):
                gx[nodes] += p[1]
                gY[c], gw[c] = p[2], p[3]
            grads = (gx, gY, gw)
        dt = time.perf_counter() - t0
    return (out,) + grads, dt


def cpu_baseline_direct(irreps, lsh, lout, wl, fwd_only, max_edges, snap=None):
    """The float64 oracle (harmonics + forward, + backward unless fwd_only) on a
    bounded sample of the workload, its edges split by receiver over a process
    pool of host_workers() workers (one BLAS thread each); per-node partial
    results are summed in the parent.  With snap (the timed step's outputs:
    out, receiver-sorted grad_Y / grad_w, grad_x, and the permutation) the
    oracle's results also give the parity of the timed run on the sample."""
    e, what = _receiver_sample(wl.src, wl.dst, max_edges)
    nodes = np.unique(np.concatenate([wl.src[e], wl.dst[e]]))
    src, dst = np.searchsorted(nodes, wl.src[e]), np.searchsorted(nodes, wl.dst[e])
    g = None if fwd_only else wl.g[nodes]
    n, W = len(nodes), host_workers()
    res, dt = pooled_oracle_direct((irreps, lsh, lout), src, dst, n, wl.x[nodes], wl.r[e], wl.w[e], g, W)
    if snap is not None:
        recv = np.unique(wl.dst[e])
        li = np.searchsorted(nodes, recv)
        checks = [("out", snap["out"][recv], res[0][li], "out")]
        if not fwd_only:
            pos = np.empty(len(snap["perm"]), dtype=np.int64)
            pos[snap["perm"]] = np.arange(len(snap["perm"]))
            checks += [("grad_Y", snap["gY"][pos[e]], res[2], "Y"), ("grad_w", snap["gw"][pos[e]], res[3], "w")]
            if len(e) == len(wl.src):        # every edge in the sample: grad_x is complete
                checks.append(("grad_x", snap["gx"][nodes], res[1], "x"))
        snap["parity"] = _parity((irreps, lsh, lout), e, len(recv), checks, what)
    return {"value": len(e) / dt, "unit": "edges/s", "cores": W, "kind": "oracle",
            "sample": f"{what}, {n} nodes: harmonics + fwd{'' if fwd_only else ' + bwd'} once, "
                      f"float64, split by receiver over {W} worker processes (1 thread each), "
                      f"{dt:.2f} s wall"}


def cpu_baseline_radial(irreps, lsh, lout, wl, radial, max_edges=30000, snap=None):
    """The float64 oracle of the radial layer (fwd + bwd with the mix) on the
    edges into the first receivers, split by receiver over the process pool
    (per-node and parameter gradients summed in the parent).  With snap (the
    timed step's mixed output, receiver-sorted grad_Y and the permutation) also
    the parity of the timed run on the sample's receivers and edges."""
    import multiprocessing as mp
    nb, _, rc = radial
    e, what = _receiver_sample(wl.src, wl.dst, max_edges)
    nodes = np.unique(np.concatenate([wl.src[e], wl.dst[e]]))
    src, dst = np.searchsorted(nodes, wl.src[e]), np.searchsorted(nodes, wl.dst[e])
    x, g, rl, r = wl.x[nodes], wl.g[nodes], wl.r_len[e], wl.r[e]
    n, W = len(nodes), host_workers()
    ctx = mp.get_context("fork")
    with ctx.Pool(W, initializer=_pool_init, initargs=((irreps, lsh, lout),)) as pool:
        pool.map(_oracle_radial_chunk, [(src[:0], dst[:0], 1, x[:1], r[:0], rl[:0], wl.W1, wl.W2, wl.Wmix,
                                         g[:1], nb, rc)] * W)
        t0 = time.perf_counter()
        tasks, maps = [], []
        for c in _chunks_by_receiver(dst, W):
            nc, ls, ld, (xc, gc) = _local(src, dst, c, x, g)
            tasks.append((ls, ld, len(nc), xc, r[c], rl[c], wl.W1, wl.W2, wl.Wmix, gc, nb, rc))
            maps.append(nc)
        parts = pool.map(_oracle_radial_chunk, tasks)
        out = np.zeros((n,) + parts[0][0].shape[1:])
        for nc, p in zip(maps, parts):
            out[nc] += p[0]
        dt = time.perf_counter() - t0
    if snap is not None:
        gY = np.zeros((len(e), parts[0][1][1].shape[1]))
        for c, p in zip(_chunks_by_receiver(dst, W), parts):
            gY[c] = p[1][1]
        recv = np.unique(wl.dst[e])
        pos = np.empty(len(snap["perm"]), dtype=np.int64)
        pos[snap["perm"]] = np.arange(len(snap["perm"]))
        checks = [("out", snap["out"][recv], out[np.searchsorted(nodes, recv)], "out"),
                  ("grad_Y", snap["gY"][pos[e]], gY, "Y")]
        snap["parity"] = _parity((irreps, lsh, lout), e, len(recv), checks, what)
    return {"value": len(e) / dt, "unit": "edges/s", "cores": W, "kind": "oracle",
            "sample": f"{what}, {n} nodes: harmonics + radial fwd + bwd with the mix once, float64, "
                      f"split by receiver over {W} worker processes (1 thread each), {dt:.2f} s wall"}


# ---------------------------------------------------------------------------
# GPU timing


def make_timers(torch, flush):
    """(do_flush, timed_steps, timed_kernel) on torch's current stream."""
    def do_flush():
        # read 1 GiB: L2 and the Infinity Cache end up holding clean lines of
        # an unrelated buffer (a write would leave dirty lines whose write-back
        # competes with the next kernel's reads)
        flush.sum()

    def timed_steps(step, k, cold):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(k)]
        for e0, e1 in ev:
            if cold:
                do_flush()
            e0.record()
            step()
            e1.record()
        torch.cuda.synchronize()
        return np.array([e0.elapsed_time(e1) for e0, e1 in ev])   # ms

    def timed_kernel(fn, copies, reps, rounds):
        # fn(c) launches on copy c of the edge-sized arrays; back-to-back
        # launches rotate over the copies, so each reads data last touched
        # `copies` launches earlier (cold when copies x bytes >= 1 GiB); the
        # duration is amortised over the batch (an event pair around a single
        # short launch mostly measures the event overhead)
        res = []
        for _ in range(rounds):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            do_flush()
            e0.record()
            for i in range(reps):
                fn(i % copies)
            e1.record()
            torch.cuda.synchronize()
            res.append(e0.elapsed_time(e1) / reps)
        return np.array(res)

    return do_flush, timed_steps, timed_kernel


def timed_stream(torch, flush, step_c, copies, k, rounds):
    # k steps back to back in one event bracket (what a training loop
    # issues), step s on copy s % copies of every array the step touches;
    # copies are chosen so that one is reused only after at least 1 GiB of
    # other data, so each step starts as cold as after a flush.  Returns
    # the per-step time of each of `rounds` brackets.
    res = []
    for _ in range(rounds):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        flush.sum()   # 1 GiB read: L2 and the Infinity Cache hold unrelated clean lines
        e0.record()
        for s in range(k):
            step_c(s % copies)
        e1.record()
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1) / k)
    return np.array(res)


def copy_bandwidth(torch, dev, flush, nbytes=1 << 29):
    """GB/s of a plain device copy (read + write of nbytes each) after a flush: the
    practical ceiling of a kernel that writes as much as it reads."""
    a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    best = None
    for _ in range(3):
        flush.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    del a, b
    return 2 * nbytes / (best * 1e-3) / 1e9


def counters_run(torch, dev, flush, step, config):
    """a few steps plus a plain 512 MiB copy (the calibration of the counters)"""
    flush.fill_(1.0)
    for _ in range(3):
        flush.sum()
        step()
    a = torch.empty(1 << 27, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    a.fill_(2.0)
    flush.sum()
    b.copy_(a)                      # plain copy: 512 MiB read + 512 MiB written
    torch.cuda.synchronize()
    print(json.dumps({"counters_run": config, "copy_bytes": a.numel() * 4}))


def hbm_roofline(kernel, nbytes, ms, traffic=None, note=None):
    gbs = nbytes / (ms * 1e-3) / 1e9
    r = {"bound": "hbm", "kernel": kernel, "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes": nbytes, "ms": ms, "traffic": traffic}
    if note:
        r["note"] = note
    return r


def node_order(g):
    """The same graph arrays without a launch order (passes walk node ids)."""
    import copy
    h = copy.copy(g)
    h.order = h.t_order = None
    return h


def bench_direct(name, args, torch, tpc, dev, flush, cpu=True):
    """One direct-weight workload: returns (result dict, step function)."""
    from workloads import CONFIGS, make_workload
    irreps, lsh, lout, desc = WORKLOADS[name]
    fwd_only = "fwd+bwd" not in CONFIGS[name]["modes"]   # the lmax-3 layer is forward only
    plan = tpc.Plan(irreps, lsh, lout)
    wl = make_workload(name, plan.dims(), seed=0)
    N, E = wl.n_nodes, wl.n_edges
    P, U, ysh = plan.n_paths, plan.mul, plan.ysh
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    src, dst = T(wl.src), T(wl.dst)
    # the graph preparation, once per neighbour list: grouping, then the
    # launch order (nodes by descending degree) every pass below walks
    g = tpc.graph_launch_order(tpc.graph_build(src, dst, N))
    Y = tpc.sph_harm(lsh, tpc.gather_rows(T(wl.r), g.perm))
    w = tpc.gather_rows(T(wl.w), g.perm)
    x = T(wl.x)
    go = None if fwd_only else T(wl.g)
    out = torch.empty(N, plan.outdim, device=dev)
    gx = torch.empty_like(x)
    NC = copies_for_cold(4 * E * (P * U + ysh))
    Ys, ws = [Y] + [Y.clone() for _ in range(NC - 1)], [w] + [w.clone() for _ in range(NC - 1)]
    gYs = [torch.empty_like(Y) for _ in range(NC)] if not fwd_only else None
    gws = [torch.empty_like(w) for _ in range(NC)] if not fwd_only else None

    # fwd+bwd signatures with a one-pass backward are also timed with their edge
    # rows in the sender grouping (tp_conv_forward_sg / tp_conv_backward_sg),
    # reported beside the step (which uses the receiver-sorted layout)
    sg = one_pass_backward(lsh) and not fwd_only
    if sg:
        e_pos = tpc.graph_sender_positions(g)
        Ygs = [tpc.gather_rows(Yc, g.t_perm) for Yc in Ys]
        wgs = [tpc.gather_rows(wc, g.t_perm) for wc in ws]

    def step():
        tpc.forward(plan, g, x, Y, w, out=out)
        if not fwd_only:
            tpc.backward(plan, g, x, Y, w, go, outs=(gx, gYs[0], gws[0]))

    if args.counters:
        if fwd_only:
            counters_run(torch, dev, flush, step, name)
        else:
            # the edge-vector step too, so the counters cover both forms
            r_c = tpc.gather_rows(T(wl.r), g.perm)
            gr_c = torch.empty_like(r_c)

            def both():
                step()
                if sg:      # the sender-grouped layout's kernels as well
                    tpc.forward_sg(plan, g, e_pos, x, Ygs[0], wgs[0], out=out)
                    tpc.backward_sg(plan, g, x, Ygs[0], wgs[0], go, outs=(gx, gYs[0], gws[0]))
                tpc.forward_r(plan, g, x, r_c, w, out=out)
                tpc.backward_r(plan, g, x, r_c, w, go, outs=(gx, gr_c, gws[0]))
            counters_run(torch, dev, flush, both, name)
        return None, step
    do_flush, timed_steps_of, timed_kernel = make_timers(torch, flush)
    timed_steps = lambda k, cold: timed_steps_of(step, k, cold)

    kernels = {"fwd": lambda c: tpc.forward(plan, g, x, Ys[c], ws[c], out=out)}
    one_pass = one_pass_backward(lsh)
    extras = {}
    if not fwd_only:
        bwd_call = lambda c: tpc.backward(plan, g, x, Ys[c], ws[c], go, outs=(gx, gYs[c], gws[c]))
        if one_pass:
            kernels["bwd"] = bwd_call
        else:
            kernels["bwd_recv"] = lambda c: tpc.backward(plan, g, x, Ys[c], ws[c], go,
                                                         outs=(None, gYs[c], gws[c]))
            kernels["bwd_send"] = lambda c: tpc.backward(plan, g, x, Ys[c], ws[c], go,
                                                         outs=(gx, None, None))
            extras["bwd"] = bwd_call
        r_sorted = tpc.gather_rows(T(wl.r), g.perm)
        grad_r = torch.empty_like(r_sorted)
        extras["forces"] = lambda c: tpc.sph_harm_backward(lsh, r_sorted, gYs[c], out=grad_r)
        # second-order backward with all three cotangents (here: the first backward's outputs)
        extras["double_bwd"] = lambda c: tpc.double_backward(plan, g, x, Ys[c], ws[c], go, gx, gYs[c],
                                                             gws[c])
        # the same step from the edge vectors: harmonics on chip, grad_r in place of grad_Y
        if sg:
            # the step's kernels with the edge rows in the sender grouping
            kernels["fwd_sg"] = lambda c: tpc.forward_sg(plan, g, e_pos, x, Ygs[c], wgs[c], out=out)
            kernels["bwd_sg"] = lambda c: tpc.backward_sg(plan, g, x, Ygs[c], wgs[c], go,
                                                          outs=(gx, gYs[c], gws[c]))
        rs = [r_sorted] + [r_sorted.clone() for _ in range(NC - 1)]
        grs = [torch.empty_like(r_sorted) for _ in range(NC)]
        geom = {"fwd_r": lambda c: tpc.forward_r(plan, g, x, rs[c], ws[c], out=out),
                "bwd_r": lambda c: tpc.backward_r(plan, g, x, rs[c], ws[c], go, outs=(gx, grs[c], gws[c]))}

    flush.fill_(1.0)
    # graph grouping, timed separately
    gb = []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        do_flush()
        e0.record()
        tpc.graph_build(src, dst, N, check=False)
        e1.record()
        torch.cuda.synchronize()
        gb.append(e0.elapsed_time(e1))
    go_ms = []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        do_flush()
        e0.record()
        tpc.graph_launch_order(g)
        e1.record()
        torch.cuda.synchronize()
        go_ms.append(e0.elapsed_time(e1))

    # Timed steps.  Where the workload is large enough that STEP_COPIES full
    # copies of everything a step touches (graph, x, Y, w, grad_out and the
    # outputs) hold at least 1 GiB, the K steps run back to back in one event
    # bracket over rotating copies (cold without a flush between steps);
    # otherwise (the 32-atom graph) each step follows a flush in its own
    # bracket.  The isolated flushed step is reported beside it either way.
    per_copy = 4 * (E * (P * U + ysh) * (1 if fwd_only else 2) + 3 * E + 2 * N
                    + N * (plan.xdim + plan.outdim) * (1 if fwd_only else 2))
    SC = 1 if per_copy >= COLD_BYTES else min(16, math.ceil(COLD_BYTES / per_copy) + 1)
    stream = max(SC - 1, 1) * per_copy >= COLD_BYTES
    stream_rounds = 3
    if stream:
        gcs = [g] + [tpc.graph_launch_order(tpc.graph_build(src, dst, N, check=False)) for _ in range(SC - 1)]
        # the same graphs walked in node order (no launch order)
        gcs_n = [node_order(gc) for gc in gcs]
        sets = [(gcs[0], x, go, out, gx)] + [
            (gcs[c], x.clone(), None if fwd_only else go.clone(), torch.empty_like(out), torch.empty_like(gx))
            for c in range(1, SC)]
        Ys_s = Ys[:SC] + [Y.clone() for _ in range(SC - len(Ys[:SC]))]
        ws_s = ws[:SC] + [w.clone() for _ in range(SC - len(ws[:SC]))]
        gYs_s = None if fwd_only else gYs[:SC] + [torch.empty_like(Y) for _ in range(SC - len(gYs[:SC]))]
        gws_s = None if fwd_only else gws[:SC] + [torch.empty_like(w) for _ in range(SC - len(gws[:SC]))]
        if sg:
            eps = [tpc.graph_sender_positions(gc) for gc in gcs]
            Ygs_s = [tpc.gather_rows(Yc, g.t_perm) for Yc in Ys_s]
            wgs_s = [tpc.gather_rows(wc, g.t_perm) for wc in ws_s]

        def step_recv(c):
            gc, xc, goc, outc, gxc = sets[c]
            tpc.forward(plan, gc, xc, Ys_s[c], ws_s[c], out=outc)
            if not fwd_only:
                tpc.backward(plan, gc, xc, Ys_s[c], ws_s[c], goc, outs=(gxc, gYs_s[c], gws_s[c]))

        def step_node_order(c):
            _, xc, goc, outc, gxc = sets[c]
            tpc.forward(plan, gcs_n[c], xc, Ys_s[c], ws_s[c], out=outc)
            if not fwd_only:
                tpc.backward(plan, gcs_n[c], xc, Ys_s[c], ws_s[c], goc, outs=(gxc, gYs_s[c], gws_s[c]))

        def step_sg(c):
            gc, xc, goc, outc, gxc = sets[c]
            tpc.forward_sg(plan, gc, eps[c], xc, Ygs_s[c], wgs_s[c], out=outc)
            tpc.backward_sg(plan, gc, xc, Ygs_s[c], wgs_s[c], goc, outs=(gxc, gYs_s[c], gws_s[c]))

    timed_steps(args.warmup, True)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    t_sg = t_no = None
    if stream:
        # brackets of the variants (node order, sender-grouped layout) and of
        # the step alternate, so none gains from its place in the run; the
        # step's own bracket comes last in each round, so the outputs read
        # back below are its (receiver-sorted) ones
        variants = [step_node_order] + ([step_sg] if sg else [])
        for f in variants + [step_recv]:
            timed_stream(torch, flush, f, SC, max(args.warmup, 1), 1)
        tv = [[] for _ in variants]
        t = []
        for _ in range(stream_rounds):
            for v, f in enumerate(variants):
                tv[v].append(timed_stream(torch, flush, f, SC, args.steps, 1)[0])
            t.append(timed_stream(torch, flush, step_recv, SC, args.steps, 1)[0])
        t = np.array(t)
        t_no = np.array(tv[0])
        t_sg = np.array(tv[1]) if sg else None
        c_last = (args.steps - 1) % SC      # the copy the last timed step wrote
        res_out, res_gx = sets[c_last][3], sets[c_last][4]
        res_gY = None if fwd_only else gYs_s[c_last]
        res_gw = None if fwd_only else gws_s[c_last]
    else:
        t = timed_steps(args.steps, True)
        res_out, res_gx = out, gx
        res_gY = None if fwd_only else gYs[0]
        res_gw = None if fwd_only else gws[0]
    torch.cuda.synchronize()
    # the timed step's results, for the parity check on the CPU-baseline sample
    snap = {"out": res_out.cpu().numpy(), "perm": g.perm.cpu().numpy()[:E]} if cpu else None
    if cpu and not fwd_only:
        snap.update(gx=res_gx.cpu().numpy(), gY=res_gY.cpu().numpy(), gw=res_gw.cpu().numpy())
    wall = time.perf_counter() - t_wall0
    t_iso = timed_steps(args.steps, True) if stream else t
    if stream:
        del sets, Ys_s, ws_s, gYs_s, gws_s
        if sg:
            del Ygs_s, wgs_s
    warm = timed_steps(args.steps, False) if args.warm else None
    reps = max(2 * NC, 12)
    rounds = max(2, args.steps // 5)
    kt = {n: float(timed_kernel(fn, NC, reps, rounds).mean()) for n, fn in kernels.items()}
    extra_ms = {n: float(timed_kernel(fn, NC, reps, rounds).mean()) for n, fn in extras.items()}
    if not fwd_only:
        def step_r():
            tpc.forward_r(plan, g, x, rs[0], ws[0], out=out)
            tpc.backward_r(plan, g, x, rs[0], ws[0], go, outs=(gx, grs[0], gws[0]))
        timed_steps_of(step_r, max(args.warmup, 1), True)
        t_r = timed_steps_of(step_r, args.steps, True)
        kt_r = {n: float(timed_kernel(fn, NC, reps, rounds).mean()) for n, fn in geom.items()}

    step_ms = float(t.mean())
    ab = algorithmic_bytes(N, E, P, U, ysh, plan.xdim, plan.outdim)
    # the dominant kernel among those of the timed step
    dom = max((n for n in kt if not n.endswith("_sg")), key=kt.get)
    traffic = read_traffic(name)
    cnt = cg_counts(plan.paths(), *plan.cg())
    fl = cg_flops(cnt)
    sb = step_bytes(ab, fwd_only)
    res = {
        "workload": f"{name}: {desc}", "n_nodes": N, "n_edges": E, "irreps": irreps,
        "lmax_sh": lsh, "lmax_out": lout, "paths": P, "mode": "fwd" if fwd_only else "fwd+bwd",
        "ms_per_step": step_ms,
        "edges_per_s": E / (step_ms * 1e-3),
        "ms_per_step_p10_p90": [float(np.percentile(t, 10)), float(np.percentile(t, 90))],
        "step_timing": (f"{args.steps} steps back to back in one event bracket, rotating over {SC} "
                        f"copies of every array a step touches ({SC * per_copy / 1e6:.0f} MB: a copy is "
                        f"reused after >= 1 GiB of other data), after a flush; mean of {stream_rounds} "
                        f"brackets" if stream else
                        f"each of {args.steps} steps after a 1 GiB flush in its own event bracket"),
        "ms_per_step_isolated": float(t_iso.mean()),
        "ms_per_step_isolated_note": ("one step after a 1 GiB flush in its own event bracket (adds the "
                                      "latency from the event to the first kernel)"),
        "fwd_edges_per_s": E / (kt["fwd"] * 1e-3),
        "kernel_ms": kt,
        "kernel_ms_note": (f"cold: {reps} back-to-back launches rotating over {NC} copies of the "
                           f"edge-sized arrays ({NC * 4 * E * (P * U + ysh) / 1e6:.0f} MB of inputs), "
                           f"after a flush; mean of {rounds}"),
        "kernel_hbm_frac": {n: ab[n] / (v * 1e-3) / 1e9 / HBM_PEAK_GBS for n, v in kt.items()},
        "roofline": hbm_roofline(dom, ab[dom], kt[dom], (traffic or {}).get(dom)),
        "step_roofline": {"bound": "hbm", "bytes": sb, "ms": step_ms,
                          "achieved": sb / (step_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                          "unit": "GB/s", "frac": sb / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                          "note": "forward + backward bytes, each array once per pass (the "
                                  "backward's re-read of w in the two-pass form is not counted)"},
        "valu_flop_util": {n: fl[n] * E * U / (v * 1e-3) / 1e12 / FP32_VALU_PEAK_TFLOPS
                           for n, v in kt.items()},
        "valu_flops_per_edge_channel": {n: fl[n] for n in kt},
        "graph_build_ms": float(np.median(gb)),
        "launch_order_ms": float(np.median(go_ms)),
        "launch_order": ("every pass launches its nodes by descending degree (tp_conv_graph_launch_order, "
                         "computed with the grouping, outside the step)"),
        "node_order_ms_per_step": None if t_no is None else float(t_no.mean()),
        "node_order_note": "the same step with the nodes launched in node order; brackets alternating",
        "wall_s_timed_region": wall,
    }
    if not fwd_only:
        res["bwd_ms"] = extra_ms.get("bwd", kt.get("bwd"))
        res["double_bwd_ms"] = extra_ms.get("double_bwd")
        res["double_bwd_hbm_frac"] = ab["double_bwd"] / (extra_ms["double_bwd"] * 1e-3) / 1e9 / HBM_PEAK_GBS
        res["double_bwd_note"] = ("second-order backward (dx, dY, dw, d grad_out for cotangents of all "
                                  "three first-order outputs), per call; not part of the step")
        res["forces_ms"] = extra_ms.get("forces")
        res["forces_note"] = ("edge-vector gradient from grad_Y (tp_conv_sph_harm_backward), per "
                              "launch; not part of the step")
        ab_r = algorithmic_bytes_geom(N, E, P, U, plan.xdim, plan.outdim)
        ms_r = float(t_r.mean())
        res["edge_vector_step"] = {
            "ms_per_step": ms_r, "edges_per_s": E / (ms_r * 1e-3), "kernel_ms": kt_r,
            "traffic": {n: (traffic or {}).get(n) for n in kt_r},
            "kernel_hbm_frac": {n: ab_r[n] / (v * 1e-3) / 1e9 / HBM_PEAK_GBS for n, v in kt_r.items()},
            "step_hbm_frac": (ab_r["fwd_r"] + ab_r["bwd_r"]) / (ms_r * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "algorithmic_bytes": ab_r,
            "note": ("forward and one-pass backward from r [E, 3]: harmonics evaluated per edge on chip, "
                     "grad_r (the forces' edge term) in place of grad_Y; timed as the step above"),
        }
    if sg:
        ms_sg = float(t_sg.mean()) if t_sg is not None else None
        res["sender_layout_step"] = {
            "ms_per_step": ms_sg, "edges_per_s": None if ms_sg is None else E / (ms_sg * 1e-3),
            "kernel_ms": {n: kt[n] for n in ("fwd_sg", "bwd_sg")},
            "kernel_hbm_frac": {n: ab[n] / (kt[n] * 1e-3) / 1e9 / HBM_PEAK_GBS for n in ("fwd_sg", "bwd_sg")},
            "traffic": {n: (traffic or {}).get(n) for n in ("fwd_sg", "bwd_sg")},
            "note": ("the step with Y, w and their gradients stored in the sender grouping: "
                     "tp_conv_forward_sg gathers the edge rows through e_pos, tp_conv_backward_sg "
                     "reads and writes them in order (results bit for bit those of the step); "
                     "timed like the step, its brackets alternating with the step's"
                     if ms_sg is not None else "kernels only (the step is timed in isolation here)"),
        }
    if warm is not None:
        res["warm_edges_per_s"] = E / (float(warm.mean()) * 1e-3)
    if cpu:
        # about 2-10 s of wall time on 16 host cores; the lmax-3 product costs
        # about 10x the lmax-2 one per edge
        res["cpu_baseline"] = cpu_baseline_direct(irreps, lsh, lout, wl, fwd_only,
                                                  max_edges=60000 if lsh <= 2 else 40000, snap=snap)
        res["parity"] = snap["parity"]
    else:
        res["cpu_baseline"] = None
        res["parity"] = None
    del Ys, ws, gYs, gws
    return res, step


def bench_radial(name, args, torch, tpc, dev, flush, cpu=True):
    """The streaming layer: returns (result dict, step function)."""
    from workloads import make_workload
    irreps, lsh, lout, radial, desc = RADIAL_WORKLOADS[name]
    plan = tpc.Plan(irreps, lsh, lout, radial=radial, uvw=True)
    wl = make_workload(name, plan.dims(), seed=0)
    N, E = wl.n_nodes, wl.n_edges
    P, U = plan.n_paths, plan.mul
    NH = radial[1]
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    src, dst = T(wl.src), T(wl.dst)
    g = tpc.graph_launch_order(tpc.graph_build(src, dst, N))    # grouping and launch order
    Y = tpc.sph_harm(lsh, tpc.gather_rows(T(wl.r), g.perm))
    rl = tpc.gather_rows(T(wl.r_len), g.perm)
    x, W1, W2, Wm, go = T(wl.x), T(wl.W1), T(wl.W2), T(wl.Wmix), T(wl.g)
    out = torch.empty(N, plan.outdim, device=dev)
    pre = torch.empty_like(out)
    outs = {"x": torch.empty_like(x), "Y": torch.empty_like(Y), "W1": torch.empty_like(W1),
            "W2": torch.empty_like(W2), "Wmix": torch.empty_like(Wm)}
    ws = torch.empty(tpc.radial_workspace(plan, N, True), dtype=torch.uint8, device=dev)

    def step():
        tpc.forward_radial(plan, g, x, Y, rl, W1, W2, Wm, out=out, out_pre=pre)
        tpc.backward_radial(plan, g, x, Y, rl, W1, W2, go, Wmix=Wm, out_pre=pre, outs=outs, ws=ws)

    if args.counters:
        counters_run(torch, dev, flush, step, name)
        return None, step
    do_flush, timed_steps, timed_kernel = make_timers(torch, flush)
    bwd = lambda want: (lambda c: tpc.backward_radial(plan, g, x, Y, rl, W1, W2, go, want=want,
                                                      outs=outs, ws=ws))
    # every launch gathers x or grad_out rows for 3M edges (GBs), far more than
    # the 256 MB Infinity Cache: one copy is cold
    kernels = {
        "fwd": lambda c: tpc.forward_radial(plan, g, x, Y, rl, W1, W2, None, out=pre),
        "bwd_recv": bwd(("Y", "W1")),
        "bwd_w2": bwd(("W2",)),
        "bwd_send": bwd(("x",)),
        "fwd_with_mix": lambda c: tpc.forward_radial(plan, g, x, Y, rl, W1, W2, Wm, out=out,
                                                     out_pre=pre),
    }
    r_sorted = tpc.gather_rows(T(wl.r), g.perm)
    grl = torch.empty_like(rl)
    grad_r = torch.empty_like(r_sorted)
    outs_f = dict(outs, rlen=grl)
    extras = {
        # receiver pass that also returns the edge-length gradient, then the
        # edge-vector gradient
        "bwd_recv_with_rlen": lambda c: tpc.backward_radial(plan, g, x, Y, rl, W1, W2, go,
                                                            want=("Y", "W1", "rlen"), outs=outs_f,
                                                            ws=ws),
        "forces": lambda c: tpc.sph_harm_backward(lsh, r_sorted, outs["Y"], grl, out=grad_r),
    }
    flush.fill_(1.0)
    timed_steps(step, args.warmup, True)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    t = timed_steps(step, args.steps, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall0
    # the same step with the nodes walked in node order (no launch order)
    gn = node_order(g)

    def step_node_order():
        tpc.forward_radial(plan, gn, x, Y, rl, W1, W2, Wm, out=out, out_pre=pre)
        tpc.backward_radial(plan, gn, x, Y, rl, W1, W2, go, Wmix=Wm, out_pre=pre, outs=outs, ws=ws)

    t_no = timed_steps(step_node_order, args.steps, True)
    step()          # the outputs read back below are the timed step's
    torch.cuda.synchronize()
    # the timed step's results, for the parity check on the CPU-baseline sample
    snap = ({"out": out.cpu().numpy(), "gY": outs["Y"].cpu().numpy(), "perm": g.perm.cpu().numpy()[:E]}
            if cpu else None)
    # the stream layer gathers GBs per call (cold without rotation); the lmax-3
    # layer's arrays fit in the Infinity Cache, so each call follows a flush
    big = E * U * 4 > (1 << 30)
    reps, rounds = (3, 2) if big else (1, 5)
    kt = {n: float(timed_kernel(fn, 1, reps, rounds).mean()) for n, fn in kernels.items()}
    extra_ms = {n: float(timed_kernel(fn, 1, reps, rounds).mean()) for n, fn in extras.items()}
    # the same step from the edge vectors: harmonics and lengths on chip, grad_r out
    outs_r = dict(outs, r=grad_r)

    def step_r():
        tpc.forward_radial_r(plan, g, x, r_sorted, W1, W2, Wm, out=out, out_pre=pre)
        tpc.backward_radial_r(plan, g, x, r_sorted, W1, W2, go, Wmix=Wm, out_pre=pre,
                              want=("x", "r", "W1", "W2", "Wmix"), outs=outs_r, ws=ws)
    timed_steps(step_r, 1, True)
    t_r = timed_steps(step_r, args.steps, True)
    kt_r = {"fwd_r": float(timed_kernel(lambda c: tpc.forward_radial_r(plan, g, x, r_sorted, W1, W2, None,
                                                                       out=pre), 1, reps, rounds).mean())}
    # second-order backward with cotangents on grad_x, grad_Y and grad_rlen (here
    # the first backward's outputs, as in a loss on forces), all outputs
    grl_c = outs_f["rlen"]
    tpc.backward_radial(plan, g, x, Y, rl, W1, W2, go, want=("x", "Y", "rlen"), outs=outs_f, ws=ws)
    d_outs = {"x": torch.empty_like(x), "Y": torch.empty_like(Y), "rlen": torch.empty_like(rl),
              "W1": torch.empty_like(W1), "W2": torch.empty_like(W2), "Wmix": torch.empty_like(Wm),
              "g": torch.empty_like(go)}
    ws2 = torch.empty(tpc.radial_double_workspace(plan, N, True), dtype=torch.uint8, device=dev)
    dbl = lambda c: tpc.double_backward_radial(plan, g, x, Y, rl, W1, W2, go, Wmix=Wm, gg_x=outs["x"],
                                               gg_Y=outs["Y"], gg_rlen=grl_c, outs=d_outs, ws=ws2)
    dbl(0)
    dbl_ms = float(timed_kernel(dbl, 1, 2, rounds).mean())
    del ws2, d_outs
    fl = radial_flops(E, P, U, NH)
    mix_flops = 2.0 * N * plan.outdim * U            # one application of the channel mix
    names = ["fwd", "bwd_recv", "bwd_w2", "bwd_send"]
    dom = max(names, key=lambda n: kt[n])
    achieved = fl[dom] / (kt[dom] * 1e-3) / 1e12
    step_ms = float(t.mean())
    step_flops = sum(fl[n] for n in names) + 3 * mix_flops   # mix forward, grad_in, grad_Wmix
    traffic = read_traffic(name, RADIAL_SOURCES[name])
    res = {
        "workload": f"{name}: {desc}", "n_nodes": N, "n_edges": E, "irreps": irreps,
        "lmax_sh": lsh, "lmax_out": lout, "paths": P,
        "radial": {"basis": radial[0], "hidden": radial[1], "r_cut": radial[2]}, "mode": "fwd+bwd",
        "ms_per_step": step_ms,
        "edges_per_s": E / (step_ms * 1e-3),
        "ms_per_step_p10_p90": [float(np.percentile(t, 10)), float(np.percentile(t, 90))],
        "launch_order": "every pass walks its nodes by descending degree (tp_conv_graph_launch_order)",
        "node_order_ms_per_step": float(t_no.mean()),
        "node_order_note": "the same step with the nodes walked in node order, one step per flush",
        "fwd_edges_per_s": E / (kt["fwd_with_mix"] * 1e-3),
        "kernel_ms": kt,
        "kernel_ms_note": ((f"per call, {reps} back-to-back calls after a cache flush, mean of {rounds} "
                            "(every call gathers GBs of node rows: cold without rotation)" if big else
                            f"one call after a cache flush, mean of {rounds}")
                           + "; bwd_recv and bwd_w2 include their partial-sum kernels"),
        "kernel_mfma_frac": {n: fl[n] / (kt[n] * 1e-3) / 1e12 / FP32_MFMA_PEAK_TFLOPS for n in names},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": achieved,
                     "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / FP32_MFMA_PEAK_TFLOPS, "algorithmic_flops": fl[dom],
                     "ms": kt[dom], "traffic": (traffic or {}).get(dom)},
        "step_roofline": {"bound": "mfma", "flops": step_flops, "ms": step_ms,
                          "achieved": step_flops / (step_ms * 1e-3) / 1e12,
                          "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                          "frac": step_flops / (step_ms * 1e-3) / 1e12 / FP32_MFMA_PEAK_TFLOPS,
                          "note": "radial-network products of the four passes plus three applications "
                                  "of the channel mix (forward, grad_in, grad_Wmix)"},
        "forces_ms": extra_ms,
        "forces_note": "receiver pass that also returns the edge-length gradient, and the "
                       "edge-vector gradient kernel; not part of the step",
        "wall_s_timed_region": wall,
    }
    dbl_flops = fl["double_bwd"] + 3 * mix_flops                  # mix: g, out_dot, d_Wmix
    res["double_bwd_ms"] = dbl_ms
    res["double_bwd_mfma_frac"] = dbl_flops / (dbl_ms * 1e-3) / 1e12 / FP32_MFMA_PEAK_TFLOPS
    res["double_bwd_note"] = ("second-order backward (d_x, d_Y, d_rlen, d_W1, d_W2, d_Wmix, d_grad_out "
                              "for cotangents on grad_x, grad_Y and grad_rlen), per call after a flush; "
                              "not part of the step; MFMA fraction on its ten network products per edge "
                              "and three applications of the mix")
    ms_r = float(t_r.mean())
    res["edge_vector_step"] = {
        "ms_per_step": ms_r, "edges_per_s": E / (ms_r * 1e-3), "kernel_ms": kt_r,
        "step_mfma_frac": step_flops / (ms_r * 1e-3) / 1e12 / FP32_MFMA_PEAK_TFLOPS,
        "note": ("forward and backward from r [E, 3] with the channel mix: harmonics and lengths "
                 "evaluated per edge on chip, grad_r (forces' edge term) in place of grad_Y; timed "
                 "as the step above"),
    }
    res["cpu_baseline"] = cpu_baseline_radial(irreps, lsh, lout, wl, radial, snap=snap) if cpu else None
    res["parity"] = snap["parity"] if cpu else None
    return res, step


def headline(name, res, args):
    """The one-line contract around a workload's result."""
    line = {
        "metric": METRIC,
        "value": res["edges_per_s"],
        "unit": "edges/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; stands in for the pages' molecular graphs and random-init models)",
        "config": {"workload": res["workload"], "n_nodes": res["n_nodes"], "n_edges": res["n_edges"],
                   "irreps": res["irreps"], "lmax_sh": res["lmax_sh"], "lmax_out": res["lmax_out"],
                   "paths": res["paths"], "mode": res["mode"],
                   "cache": res.get("step_timing", "L2+MALL flushed before each step") +
                            "; kernels cold by rotating copies"},
    }
    line.update({k: v for k, v in res.items() if k not in ("workload", "n_nodes", "n_edges", "irreps",
                                                           "lmax_sh", "lmax_out", "paths", "mode",
                                                           "ms_per_step", "edges_per_s")})
    return line


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="all",
                    choices=["all"] + sorted(WORKLOADS) + sorted(RADIAL_WORKLOADS) + sorted(FC_WORKLOADS)
                    + sorted(GAUNT_WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--warm", action="store_true",
                    help="also time the steps back to back without the cache flush")
    ap.add_argument("--counters", action="store_true",
                    help="short run for rocprofv3 counter passes: a few steps plus a 512 MiB copy")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(the receiver-range sharding is a design, not code). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import tensor_product_convolution_amd as tpc

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.config in FC_WORKLOADS:
        return bench_fc(args, torch, tpc, dev)
    if args.config in GAUNT_WORKLOADS:
        return bench_gaunt(args, torch, tpc, dev)
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
    cpu = not args.no_cpu_baseline
    name = "mid" if args.config == "all" else args.config
    if name in RADIAL_WORKLOADS:
        res, _ = bench_radial(name, args, torch, tpc, dev, flush, cpu)
    else:
        res, _ = bench_direct(name, args, torch, tpc, dev, flush, cpu)
    if res is None:          # counters run
        return
    line = headline(name, res, args)
    line["copy_GBs"] = copy_bandwidth(torch, dev, flush)
    line["copy_note"] = ("plain device copy of 512 MiB (read + write) after a flush: the practical "
                         "ceiling of a kernel that writes as much as it reads")
    if args.config == "all":
        configs = {}
        for other in DEFAULT_CONFIGS:
            torch.cuda.empty_cache()
            if other in RADIAL_WORKLOADS:
                r, _ = bench_radial(other, args, torch, tpc, dev, flush, cpu)
            else:
                r, _ = bench_direct(other, args, torch, tpc, dev, flush, cpu)
            configs[other] = r
            print(json.dumps({"progress": other, "ms_per_step": r["ms_per_step"]}), file=sys.stderr,
                  flush=True)
        line["configs"] = configs
    print(json.dumps(line))


def fc_algorithmic(N, E, P, U, H, d3_paths, d1_paths, xdim, outdim, ysh):
    """Bytes each phase of the fully connected layer must move once, counting
    the node-sized states it writes and reads back (the reassociated schedule's
    own traffic): S and gS have H U sum_p (2l3+1) floats per node, Q has
    H U sum_p (2l1+1)."""
    s_state = 4.0 * N * H * U * sum(d3_paths)
    q_state = 4.0 * N * H * U * sum(d1_paths)
    edge_in = 4.0 * E * (1 + ysh + H)                  # col (or t_perm / t_col), Y, R
    theta = 4.0 * H * P * U * U
    node = 4.0 * N * (xdim + outdim)
    return {
        "fwd": edge_in + node + theta + 2 * s_state,
        "bwd_theta": 4.0 * N * outdim + theta + s_state,   # the forward's saved S read once
        "bwd_RY": edge_in + 4.0 * N * (xdim + outdim) + theta + 2 * s_state + 4.0 * E * (ysh + H),
        "bwd_x": edge_in + 4.0 * E + 4.0 * N * (outdim + xdim) + theta + 2 * q_state,
        "compulsory": 4.0 * E * (1 + 2 * ysh + 2 * H) + 4.0 * N * 2 * (xdim + outdim) + 2 * theta,
    }


def bench_fc(args, torch, tpc, dev):
    from workloads import make_fc_inputs, make_workload
    irreps, lsh, lout, H, desc = FC_WORKLOADS[args.config]
    plan = tpc.Plan(irreps, lsh, lout)
    wl = make_workload("mid", plan.dims(), seed=0)
    N, E = wl.n_nodes, wl.n_edges
    P, U = plan.n_paths, plan.mul
    R, Th = make_fc_inputs(E, P, U, H, seed=0)
    go_h = np.random.default_rng(1).normal(size=(N, plan.outdim)).astype(np.float32)
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    g = tpc.graph_build(T(wl.src), T(wl.dst), N)
    Y = tpc.sph_harm(lsh, tpc.gather_rows(T(wl.r), g.perm))
    Rs = tpc.gather_rows(T(R), g.perm)
    x, Tht, go = T(wl.x), T(Th), T(go_h)
    out = torch.empty(N, plan.outdim, device=dev)
    # one workspace for both calls: the backward reads the state the forward left in it
    ws = torch.empty(tpc.fc_backward_workspace(plan, N, H), dtype=torch.uint8, device=dev)
    wsb = ws
    gx, gY, gR, gT = torch.empty_like(x), torch.empty_like(Y), torch.empty_like(Rs), torch.empty_like(Tht)
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)

    def step():
        tpc.forward_fc(plan, g, x, Y, Rs, Tht, out=out, ws=ws)
        tpc.backward_fc(plan, g, x, Y, Rs, Tht, go, ws=wsb, outs=(gx, gY, gR, gT), state_saved=True)

    phases = {
        "fwd": lambda: tpc.forward_fc(plan, g, x, Y, Rs, Tht, out=out, ws=ws),
        "bwd_theta": lambda: tpc.backward_fc(plan, g, x, Y, Rs, Tht, go, ws=wsb, outs=(None, None, None, gT),
                                             state_saved=True),
        "bwd_RY": lambda: tpc.backward_fc(plan, g, x, Y, Rs, Tht, go, ws=wsb, outs=(None, gY, gR, None)),
        "bwd_x": lambda: tpc.backward_fc(plan, g, x, Y, Rs, Tht, go, ws=wsb, outs=(gx, None, None, None)),
    }
    if args.counters:
        counters_run(torch, dev, flush, step, args.config)
        return
    do_flush, timed_steps, timed_kernel = make_timers(torch, flush)
    flush.fill_(1.0)
    timed_steps(step, args.warmup, True)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    t = timed_steps(step, args.steps, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall0
    step_ms = float(np.median(t))
    # the timed step's results (forward output, receiver-sorted grad_Y and grad_R)
    snap = (dict(out=out.cpu().numpy(), gY=gY.cpu().numpy(), gR=gR.cpu().numpy(), perm=g.perm.cpu().numpy()[:E])
            if not args.no_cpu_baseline else None)
    reps, rounds = 5, max(2, args.steps // 5)
    kt = {n: float(timed_kernel(lambda c, f=fn: f(), 1, reps, rounds).mean()) for n, fn in phases.items()}
    # second-order backward, all four cotangents (here the first backward's outputs)
    tpc.backward_fc(plan, g, x, Y, Rs, Tht, go, ws=wsb, outs=(gx, gY, gR, gT))
    wsd = torch.empty(tpc.fc_double_workspace(plan, N, E, H), dtype=torch.uint8, device=dev)
    dbl = lambda c: tpc.double_backward_fc(plan, g, x, Y, Rs, Tht, go, gg_x=gx, gg_Y=gY, gg_R=gR, gg_Theta=gT,
                                           ws=wsd)
    dbl(0)
    dbl_ms = float(timed_kernel(dbl, 1, 3, rounds).mean())
    d3s = [2 * l3 + 1 for (_, _, l3, _) in plan.paths()]
    d1s = [2 * l1 + 1 for (l1, _, _, _) in plan.paths()]
    alg = fc_algorithmic(N, E, P, U, H, d3s, d1s, plan.xdim, plan.outdim, plan.ysh)
    dom = max(kt, key=kt.get)
    gbs = alg[dom] / (kt[dom] * 1e-3) / 1e9
    res = {
        "metric": METRIC, "value": E / (step_ms * 1e-3), "unit": "edges/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": step_ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded; random radial features, mixing parameters and upstream gradient)",
        "config": {"workload": f"{args.config}: {desc}", "n_nodes": N, "n_edges": E,
                   "irreps": irreps, "paths": P, "radial_features": H, "mode": "fwd+bwd",
                   "cache": "L2+MALL flushed before each step"},
        "ms_per_step_p10_p90": [float(np.percentile(t, 10)), float(np.percentile(t, 90))],
        "phase_ms": kt,
        "fwd_edges_per_s": E / (kt["fwd"] * 1e-3),
        "compulsory_bytes": alg["compulsory"],
        "state_bytes": tpc.fc_workspace(plan, N, H),
        "backward_note": "the backward reads the state S the forward left in the shared workspace "
                         "(TP_FC_STATE_SAVED) instead of recomputing it",
        "double_bwd_ms": dbl_ms,
        "double_bwd_note": "second-order backward with cotangents on all four first-order outputs "
                           "(four reassociated forwards and four backwards, one operand replaced in each); "
                           "per call after a flush, not part of the step",
        "wall_s_timed_region": wall,
        "roofline": {"bound": "hbm", "kernel": f"{dom} (one entry-point call)",
                     "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes": alg[dom],
                     "note": "inputs and outputs once plus one write and one read of each "
                             "node-sized state the phase uses", "traffic": None},
        "cpu_baseline": None,
        "parity": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        op = oracle.build_plan(irreps, lsh, lout)
        from threadpoolctl import threadpool_limits
        e, what = _receiver_sample(wl.src, wl.dst, 12000)
        nodes = np.unique(np.concatenate([wl.src[e], wl.dst[e]]))
        src, dst = np.searchsorted(nodes, wl.src[e]), np.searchsorted(nodes, wl.dst[e])
        with threadpool_limits(1):
            t0 = time.perf_counter()
            Yo = oracle.sh_real(lsh, wl.r[e])
            ro = oracle.fc_conv_fwd(op, src, dst, len(nodes), wl.x[nodes], Yo, R[e], Th)
            rb = oracle.fc_conv_bwd(op, src, dst, len(nodes), wl.x[nodes], Yo, R[e], Th, go_h[nodes])
            dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": len(e) / dt, "unit": "edges/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{what}, harmonics + fwd + bwd once, float64 (per-edge "
                                         f"weights formed), one process with one BLAS thread, {dt:.2f} s"}
        recv = np.unique(wl.dst[e])
        pos = np.empty(E, dtype=np.int64)
        pos[snap["perm"]] = np.arange(E)
        res["parity"] = _parity((irreps, lsh, lout), e, len(recv), [
            ("out", snap["out"][recv], ro[np.searchsorted(nodes, recv)], "out"),
            ("grad_Y", snap["gY"][pos[e]], rb[1], "Y"),
            ("grad_R", snap["gR"][pos[e]], rb[2], "all")], what)
    print(json.dumps(res))


def gaunt_algorithmic(N, E, U, xdim, ysh, wdim, outdim):
    """Per kernel of the Gaunt step: compulsory bytes (each array it must touch
    once) and the fp32 matrix-core flops it issues (32x32x2 products of 4,096
    flops per 32-channel tile): forward f = x Yq (5) and g = w Z (2) per edge;
    receiver backward f (5) per edge plus gH (5) per receiver; sender backward
    gH (5) and g (2) per edge."""
    tiles = max(1, U // 32)
    fl = 2.0 * 32 * 32 * 2 * tiles
    edge_in = 4.0 * E * (1 + ysh + wdim)            # col (or t_perm / t_col), Y, w
    return {
        "fwd": {"bytes": edge_in + 4.0 * (N + 1 + N * (xdim + outdim)), "flops": fl * 7 * E},
        "bwd_recv": {"bytes": edge_in + 4.0 * E * (ysh + wdim) + 4.0 * (N + 1 + N * (xdim + outdim)),
                     "flops": fl * (5 * E + 5 * N)},
        "bwd_send": {"bytes": 4.0 * E * (2 + ysh + wdim) + 4.0 * (N + 1 + N * (xdim + outdim)),
                     "flops": fl * 7 * E},
        "step_bytes": 4.0 * E * (1 + 2 * ysh + 2 * wdim) + 4.0 * (N + 1 + 2 * N * (xdim + outdim)),
    }


def bench_gaunt(args, torch, tpc, dev):
    from workloads import make_gaunt_weights, make_workload
    irreps, lsh, lout, desc = GAUNT_WORKLOADS[args.config]
    plan = tpc.Plan(irreps, lsh, lout, mode=tpc.TP_MODE_GAUNT)
    outdim, wdim, Q = tpc.gaunt_dims(plan)
    U = plan.mul
    dims = dict(xdim=plan.xdim, n_paths=1, U=U, outdim=outdim, n_out_irreps=lout + 1)
    wl = make_workload("mid", dims, seed=0)
    N, E = wl.n_nodes, wl.n_edges
    w = make_gaunt_weights(E, lsh, U, seed=0)
    go_h = np.random.default_rng(1).normal(size=(N, outdim)).astype(np.float32)
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    g = tpc.graph_build(T(wl.src), T(wl.dst), N)
    Y = tpc.sph_harm(lsh, tpc.gather_rows(T(wl.r), g.perm))
    ws_ = tpc.gather_rows(T(w.reshape(E, -1)), g.perm)
    x, go = T(wl.x), T(go_h)
    out = torch.empty(N, outdim, device=dev)
    gx, gY, gw = torch.empty_like(x), torch.empty_like(Y), torch.empty_like(ws_)
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)

    def step():
        tpc.forward_gaunt(plan, g, x, Y, ws_, out=out)
        tpc.backward_gaunt(plan, g, x, Y, ws_, go, outs=(gx, gY, gw))

    kernels = {
        "fwd": lambda: tpc.forward_gaunt(plan, g, x, Y, ws_, out=out),
        "bwd_recv": lambda: tpc.backward_gaunt(plan, g, x, Y, ws_, go, outs=(None, gY, gw)),
        "bwd_send": lambda: tpc.backward_gaunt(plan, g, x, Y, ws_, go, outs=(gx, None, None)),
    }
    if args.counters:
        counters_run(torch, dev, flush, step, args.config)
        return
    do_flush, timed_steps, timed_kernel = make_timers(torch, flush)
    flush.fill_(1.0)
    timed_steps(step, args.warmup, True)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    t = timed_steps(step, args.steps, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall0
    step_ms = float(np.median(t))
    # the timed step's results (receiver-sorted grad_Y and grad_w)
    snap = (dict(out=out.cpu().numpy(), gx=gx.cpu().numpy(), gY=gY.cpu().numpy(), gw=gw.cpu().numpy(),
                 perm=g.perm.cpu().numpy()[:E]) if not args.no_cpu_baseline else None)
    reps, rounds = 10, max(2, args.steps // 5)
    kt = {n: float(timed_kernel(lambda c, f=fn: f(), 1, reps, rounds).mean()) for n, fn in kernels.items()}
    # second-order backward, all three cotangents (here the first backward's outputs)
    tpc.backward_gaunt(plan, g, x, Y, ws_, go, outs=(gx, gY, gw))
    wsd = torch.empty(tpc.gaunt_double_workspace(plan, N, E), dtype=torch.uint8, device=dev)
    dbl = lambda c: tpc.double_backward_gaunt(plan, g, x, Y, ws_, go, gg_x=gx, gg_Y=gY, gg_w=gw, ws=wsd)
    dbl(0)
    dbl_ms = float(timed_kernel(dbl, 1, 3, rounds).mean())
    alg = gaunt_algorithmic(N, E, U, plan.xdim, plan.ysh, wdim, outdim)
    dom = max(kt, key=kt.get)
    tfs = alg[dom]["flops"] / (kt[dom] * 1e-3) / 1e12
    traffic = (read_traffic(args.config, GAUNT_SOURCES) or {}).get("gaunt_" + dom)
    res = {
        "metric": METRIC, "value": E / (step_ms * 1e-3), "unit": "edges/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": step_ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded; mid graph, random filter weights and upstream gradient)",
        "config": {"workload": f"{args.config}: {desc}", "n_nodes": N, "n_edges": E,
                   "irreps": irreps, "out_irreps": plan.out_irreps, "grid_points": Q,
                   "weights_per_edge": wdim, "mode": "fwd+bwd",
                   "cache": "L2+MALL flushed before each step"},
        "ms_per_step_p10_p90": [float(np.percentile(t, 10)), float(np.percentile(t, 90))],
        "kernel_ms": kt,
        "fwd_edges_per_s": E / (kt["fwd"] * 1e-3),
        "double_bwd_ms": dbl_ms,
        "double_bwd_note": "second-order backward with cotangents on all three first-order outputs "
                           "(three grid forwards and three grid backwards, one operand replaced in each); "
                           "per call after a flush, not part of the step",
        "compulsory_bytes": alg["step_bytes"],
        "hbm_frac_step": alg["step_bytes"] / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "hbm_frac_per_kernel": {n: alg[n]["bytes"] / (kt[n] * 1e-3) / 1e9 / HBM_PEAK_GBS for n in kt},
        "wall_s_timed_region": wall,
        "roofline": {"bound": "mfma", "kernel": dom,
                     "achieved": tfs, "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tfs / FP32_MFMA_PEAK_TFLOPS, "algorithmic_flops": alg[dom]["flops"],
                     "note": "fp32 matrix-core flops the kernel issues (signals on the grid); its "
                             "compulsory bytes are in hbm_frac_per_kernel",
                     "traffic": traffic},
        "cpu_baseline": None,
        "parity": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        from threadpoolctl import threadpool_limits
        gp = oracle.gaunt_plan(irreps, lsh, lout)
        dts = []
        with threadpool_limits(1):
            for _ in range(3):
                t0 = time.perf_counter()
                Yo = oracle.sh_real(lsh, wl.r)
                ro = oracle.gaunt_conv_fwd(gp, wl.src, wl.dst, N, wl.x, Yo, w)
                rb = oracle.gaunt_conv_bwd(gp, wl.src, wl.dst, N, wl.x, Yo, w, go_h)
                dts.append(time.perf_counter() - t0)
        dt = float(np.median(dts))
        pos = np.empty(E, dtype=np.int64)
        pos[snap["perm"]] = np.arange(E)
        Ug = gp.U
        blocks = {"out": [slice(Ug * l * l, Ug * (l + 1) ** 2) for l in range(lout + 1)],
                  "x": [slice(o, o + Ug * (2 * l + 1)) for l, o in zip(gp.degrees, gp.in_offsets)],
                  "Y": [slice(l * l, (l + 1) ** 2) for l in range(lsh + 1)],
                  "w": [slice(l * Ug, (l + 1) * Ug) for l in range(lsh + 1)]}
        res["parity"] = _parity(None, None, N, [
            ("out", snap["out"], ro, "out"), ("grad_x", snap["gx"], rb[0], "x"),
            ("grad_Y", snap["gY"][pos], rb[1], "Y"), ("grad_w", snap["gw"][pos], rb[2], "w")],
            f"the whole workload ({E} edges)", blocks=blocks)
        res["cpu_baseline"] = {"value": E / dt, "unit": "edges/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"the whole workload ({E} edges), harmonics + Gaunt fwd + bwd, "
                                         f"float64, one process with one BLAS thread, median of 3 runs "
                                         f"({dt:.2f} s each)"}
    print(json.dumps(res))


if __name__ == "__main__":
    main()
