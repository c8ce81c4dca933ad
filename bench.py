"""Throughput of the fused tensor-product convolution on one MI355X.

A step is one pass of the hot path over one batch: the forward kernel, the
backward receiver pass (grad_w, grad_Y) and the backward sender pass
(grad_x), on the 1,536-atom / 46,080-edge workload (32x0e+32x1o+32x2e,
harmonics to l = 2, every path with l3 <= 2, channel-wise weights) by
default.  The graph grouping (CSR build) is timed separately: it runs once per
neighbour list, not per layer.

Timing: W untimed warm-up steps, then K timed steps, each bracketed by a pair
of HIP events on the stream the kernels run on (torch's current stream).
Before each step a 1 GiB buffer is read so that L2 and the 256 MB Infinity
Cache hold none of the step's inputs: they come from HBM.  Per-kernel launch
durations (for the roofline) are event-timed over 10 back-to-back launches of
that kernel after a flush.  ``--warm`` also times steps without the flush.

``--config stream`` times the 100,000-atom / 3,000,000-edge streaming layer
instead: edge weights from the radial network (8 Bessel functions, 64 SiLU
units, 15 x 128 weights per edge) recomputed on chip in every pass, then the
128 x 128 channel mix per output irrep; a step is its forward (radial pass +
mix) and backward (mix adjoint, receiver pass, grad_W2 pass, sender pass).
Its kernels are bound by the fp32 MFMA work of the radial network, so its
roofline is reported against the 157.3 TFLOP/s fp32 matrix peak.

Output: one JSON line (rank 0, N = 1).  ``value`` is edges per second of
forward + backward; ``roofline`` reports the slowest of the three kernels
against the 8 TB/s HBM peak with its algorithmic bytes; ``cpu_baseline`` is
the float64 oracle timed on this host's cores on the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TP-conv edges/sec (fwd, fwd+bwd) fp32 at 1 GPU; % of MI355X HBM roofline"
HBM_PEAK_GBS = 8000.0
WORKLOADS = {
    "mid": ("32x0e+32x1o+32x2e", 2, 2,
            "1536 atoms, 46080 directed edges (30 distinct random senders each), "
            "32x0e+32x1o+32x2e, real SH lmax 2, all paths l3<=2 (15), uvu weights, fwd+bwd"),
    "tiny": ("8x0e+8x1o", 2, 2, "32 atoms in an 8 A periodic cube, cutoff 4 A, 8x0e+8x1o"),
    "lmax3": ("64x0e+64x1o+64x2e+64x3o", 3, 3, "4096 atoms, degree U{5..30}, lmax 3, 64 channels"),
    "zipf": ("64x0e+64x1o+64x2e+64x3o", 3, 3,
             "32768 atoms, Zipf(1.5) degrees capped at 256, lmax 3, 64 channels"),
}
RADIAL_WORKLOADS = {
    "stream": ("128x0e+128x1o+128x2e", 2, 2, (8, 64, 5.0),
               "100000 atoms, 3000000 directed edges (30 distinct random senders each, length "
               "U[0.8,5] A), 128x0e+128x1o+128x2e, real SH lmax 2, all paths l3<=2 (15), edge "
               "weights from a radial MLP (8 Bessel -> 64 SiLU -> 15x128) computed on chip, "
               "128x128 uvw mix per output irrep, fwd+bwd"),
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
GAUNT_SOURCES = ("gaunt.hip",)
FP32_MFMA_PEAK_TFLOPS = 157.3
PROFILE_SUMMARY = os.path.join(ROOT, "profiles", "hbm_traffic_{}.txt")
KERNEL_SOURCES = ("conv_kernels.hpp", "sig.hpp", "cg_table.hpp")
RADIAL_SOURCES = ("radial_kernels.hpp", "radial_l012_s2.hip", "uvw.hip", "conv_kernels.hpp", "sig.hpp",
                  "cg_table.hpp")
FC_SOURCES = ("fc_kernels.hip", "radial_kernels.hpp", "conv_kernels.hpp", "sig.hpp", "cg_table.hpp")


def kernel_source_hash(sources=KERNEL_SOURCES):
    h = hashlib.sha256()
    d = os.path.join(ROOT, "tensor_product_convolution_amd", "csrc")
    for f in sources:
        h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def algorithmic_bytes(N, E, P, U, ysh, xdim, outdim):
    """Bytes each kernel must move at least once (node arrays once, edge streams once)."""
    node = 4 * N * (xdim + outdim + 1)        # x, out (or grad_out / grad_x), row pointers
    return {
        "fwd": E * (4 * P * U + 4 * ysh + 4) + node,          # w, Y, col in; out
        "bwd_recv": E * (8 * P * U + 8 * ysh + 4) + node,     # w, Y, col in; grad_w, grad_Y out
        "bwd_send": E * (4 * P * U + 4 * ysh + 8) + node,     # w, Y, t_perm, t_col in; grad_x out
        # compulsory bytes of the whole step: each array once
        "step": E * (8 * P * U + 8 * ysh + 4) + 4 * N * (2 * xdim + 2 * outdim + 1),
        # second-order backward, each array once: w, gg_w, Y, gg_Y, col, t_perm,
        # t_col in, d_w and d_Y out; x, gg_x, grad_out and both row pointers in,
        # d_x and d_grad_out out
        "double_bwd": E * (12 * P * U + 12 * ysh + 12) + 4 * N * (3 * xdim + 2 * outdim + 2),
    }


def radial_flops(E, P, U, NH):
    """MFMA flops per launch: each pass forms [E x NH] x [NH x P*U] products."""
    mlp = 2.0 * NH * P * U * E
    return {"fwd": mlp, "bwd_recv": 2 * mlp, "bwd_w2": mlp, "bwd_send": mlp}


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


def cpu_baseline(op, wl, fwd_only=False, max_edges=60000):
    """The float64 oracle on this host: harmonics + fwd (+ bwd) over the whole
    workload, or over the edges into the first receivers when it has more than
    max_edges edges (a bounded sample of the same graph)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = 1
    src, dst, r, n, x, g = wl.src, wl.dst, wl.r, wl.n_nodes, wl.x, wl.g
    w = wl.w
    what = f"whole workload ({wl.n_edges} edges)"
    if wl.n_edges > max_edges:
        order = np.argsort(dst, kind="stable")
        e = np.sort(order[:max_edges])
        e = e[np.isin(dst[e], np.unique(dst[order[:max_edges]])[:-1])]   # whole receivers only
        nodes = np.unique(np.concatenate([src[e], dst[e]]))
        src, dst = np.searchsorted(nodes, src[e]), np.searchsorted(nodes, dst[e])
        r, w, x, n = r[e], w[e], x[nodes], len(nodes)
        g = None if g is None else g[nodes]
        what = (f"edges into the first receivers ({len(e)} of {wl.n_edges} edges, "
                f"{n} nodes)")
    t0 = time.perf_counter()
    Y = oracle.sh_real(op.lmax_sh, r)
    oracle.tp_conv_fwd(op, src, dst, n, x, Y, w)
    if not fwd_only:
        oracle.tp_conv_bwd(op, src, dst, n, x, Y, w, g)
    dt = time.perf_counter() - t0
    return {"value": len(src) / dt, "unit": "edges/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{what}, harmonics + fwd{'' if fwd_only else ' + bwd'} once, float64, "
                      f"{dt:.2f} s; host affinity {len(os.sched_getaffinity(0))} cores"}


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

    def timed_kernel(fn, reps, rounds):
        # launch duration amortised over back-to-back launches (an event pair
        # around a single short launch mostly measures the event overhead)
        res = []
        for _ in range(rounds):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            do_flush()
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            res.append(e0.elapsed_time(e1) / reps)
        return np.array(res)

    return do_flush, timed_steps, timed_kernel


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="mid",
                    choices=sorted(WORKLOADS) + sorted(RADIAL_WORKLOADS) + sorted(FC_WORKLOADS)
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
    from workloads import make_workload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.config in RADIAL_WORKLOADS:
        return bench_radial(args, torch, tpc, make_workload, dev)
    if args.config in FC_WORKLOADS:
        return bench_fc(args, torch, tpc, make_workload, dev)
    if args.config in GAUNT_WORKLOADS:
        return bench_gaunt(args, torch, tpc, make_workload, dev)
    irreps, lsh, lout, desc = WORKLOADS[args.config]
    from workloads import CONFIGS
    fwd_only = "fwd+bwd" not in CONFIGS[args.config]["modes"]   # the lmax-3 layer is forward only
    plan = tpc.Plan(irreps, lsh, lout)
    wl = make_workload(args.config, plan.dims(), seed=0)
    N, E = wl.n_nodes, wl.n_edges
    P, U, ysh = plan.n_paths, plan.mul, plan.ysh
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    src, dst = T(wl.src), T(wl.dst)
    g = tpc.graph_build(src, dst, N)
    Y = tpc.sph_harm(lsh, tpc.gather_rows(T(wl.r), g.perm))
    w = tpc.gather_rows(T(wl.w), g.perm)
    x = T(wl.x)
    go = None if fwd_only else T(wl.g)
    out = torch.empty(N, plan.outdim, device=dev)
    gx = torch.empty_like(x)
    gY = torch.empty_like(Y)
    gw = torch.empty_like(w)
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB

    def step():
        tpc.forward(plan, g, x, Y, w, out=out)
        if not fwd_only:
            tpc.backward(plan, g, x, Y, w, go, outs=(gx, gY, gw))   # receiver, then sender pass

    if args.counters:
        counters_run(torch, dev, flush, step, args.config)
        return
    do_flush, timed_steps_of, timed_kernel = make_timers(torch, flush)
    timed_steps = lambda k, cold: timed_steps_of(step, k, cold)

    kernels = {"fwd": lambda: tpc.forward(plan, g, x, Y, w, out=out)}
    extras = {}
    if not fwd_only:
        kernels["bwd_recv"] = lambda: tpc.backward(plan, g, x, Y, w, go, outs=(None, gY, gw))
        kernels["bwd_send"] = lambda: tpc.backward(plan, g, x, Y, w, go, outs=(gx, None, None))
        extras["bwd"] = lambda: tpc.backward(plan, g, x, Y, w, go, outs=(gx, gY, gw))
        r_sorted = tpc.gather_rows(T(wl.r), g.perm)
        grad_r = torch.empty_like(r_sorted)
        extras["forces"] = lambda: tpc.sph_harm_backward(lsh, r_sorted, gY, out=grad_r)
        # second-order backward with all three cotangents (here: the first backward's outputs)
        extras["double_bwd"] = lambda: tpc.double_backward(plan, g, x, Y, w, go, gx, gY, gw)

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

    timed_steps(args.warmup, True)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    t = timed_steps(args.steps, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall0
    warm = timed_steps(args.steps, False) if args.warm else None
    reps, rounds = 10, max(2, args.steps // 5)
    kt_all = {n: timed_kernel(fn, reps, rounds) for n, fn in kernels.items()}
    extra_ms = {n: float(timed_kernel(fn, reps, rounds).mean()) for n, fn in extras.items()}

    names = list(kernels)
    kt = np.array([kt_all[n].mean() for n in names])     # ms per launch
    copy_gbs = copy_bandwidth(torch, dev, flush)
    wk = read_profile_value(args.config, "write_kib.fwd", KERNEL_SOURCES)
    fwd_write_ratio = None if wk is None else wk * 1024 / (4.0 * N * plan.outdim)
    step_ms = float(t.mean())
    fwd_ms = float(kt[0])
    ab = algorithmic_bytes(N, E, P, U, ysh, plan.xdim, plan.outdim)
    dom = names[int(np.argmax(kt))]
    dom_ms = float(kt[names.index(dom)])
    achieved = ab[dom] / (dom_ms * 1e-3) / 1e9
    traffic = read_traffic(args.config)
    res = {
        "metric": METRIC,
        "value": E / (step_ms * 1e-3),
        "unit": "edges/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; stands in for the pages' molecular graph)",
        "config": {"workload": f"{args.config}: {desc}", "n_nodes": N, "n_edges": E,
                   "irreps": irreps, "lmax_sh": lsh, "lmax_out": lout, "paths": P,
                   "mode": "fwd" if fwd_only else "fwd+bwd",
                   "cache": "L2+MALL flushed before each step"},
        "fwd_edges_per_s": E / (fwd_ms * 1e-3),
        "fwd_edges_per_s_note": "forward kernel alone (launch duration); value is the whole step",
        "ms_per_step_p10_p90": [float(np.percentile(t, 10)), float(np.percentile(t, 90))],
        "kernel_ms": {n: float(v) for n, v in zip(names, kt)},
        "kernel_ms_note": f"per launch, {reps} back-to-back launches after a cache flush, mean of {rounds}",
        "kernel_hbm_frac": {n: ab[n] / (float(v) * 1e-3) / 1e9 / HBM_PEAK_GBS for n, v in zip(names, kt)},
        "bwd_ms": extra_ms.get("bwd"),
        "bwd_note": "one backward call (receiver then sender pass), per call",
        "double_bwd_ms": extra_ms.get("double_bwd"),
        "double_bwd_hbm_frac": (None if "double_bwd" not in extra_ms else
                                ab["double_bwd"] / (extra_ms["double_bwd"] * 1e-3) / 1e9 / HBM_PEAK_GBS),
        "double_bwd_note": "second-order backward (dx, dY, dw, d grad_out for cotangents of all "
                           "three first-order outputs), per call; not part of the step",
        "forces_ms": extra_ms.get("forces"),
        "forces_note": "edge-vector gradient from grad_Y (tp_conv_sph_harm_backward), per launch; "
                       "not part of the step",
        "step_hbm_frac": ab["fwd" if fwd_only else "step"] / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "copy_GBs": copy_gbs,
        "copy_note": "plain device copy of 512 MiB (read + write) after a flush: the practical "
                     "ceiling of a kernel that writes as much as it reads",
        "fwd_write_ratio": fwd_write_ratio,
        "fwd_write_note": "forward HBM writes (rocprofv3 WRITE_SIZE, committed summary) over "
                          "N*outdim*4: 1.0 means nothing but the output is written",
        "warm_edges_per_s": None if warm is None else E / (float(warm.mean()) * 1e-3),
        "graph_build_ms": float(np.median(gb)),
        "wall_s_timed_region": wall,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "algorithmic_bytes": ab[dom],
                     "traffic": (traffic or {}).get(dom)},
    }
    if not args.no_cpu_baseline:
        import oracle
        op = oracle.build_plan(irreps, lsh, lout)
        # about 10-30 s of oracle work: the lmax-3 product costs ~10x the lmax-2 one per edge
        res["cpu_baseline"] = cpu_baseline(op, wl, fwd_only, max_edges=60000 if lsh <= 2 else 12000)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res))


def cpu_baseline_radial(op, wl, radial, n_recv=200):
    """The float64 oracle on this host, fwd + bwd (with the mix) over the edges
    into the first n_recv receivers (a bounded sample of the layer)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = 1
    nb, _, rc = radial
    recv = np.arange(n_recv)
    e = np.nonzero(np.isin(wl.dst, recv))[0]
    nodes = np.unique(np.concatenate([wl.src[e], recv]))
    src, dst = np.searchsorted(nodes, wl.src[e]), np.searchsorted(nodes, wl.dst[e])
    x, g, rl = wl.x[nodes], wl.g[nodes], wl.r_len[e]
    t0 = time.perf_counter()
    Y = oracle.sh_real(op.lmax_sh, wl.r[e])
    oracle.tp_conv_radial_fwd(op, src, dst, len(nodes), x, Y, rl, wl.W1, wl.W2, wl.Wmix, nb, rc)
    oracle.tp_conv_radial_bwd(op, src, dst, len(nodes), x, Y, rl, wl.W1, wl.W2, wl.Wmix, g, nb, rc)
    dt = time.perf_counter() - t0
    return {"value": len(e) / dt, "unit": "edges/s", "cores": int(threads), "kind": "oracle",
            "sample": f"edges into receivers 0..{n_recv - 1} ({len(e)} of {wl.n_edges} edges, "
                      f"{len(nodes)} nodes): harmonics + radial fwd + bwd with the mix once, "
                      f"float64, {dt:.2f} s; host affinity {len(os.sched_getaffinity(0))} cores"}


def bench_radial(args, torch, tpc, make_workload, dev):
    irreps, lsh, lout, radial, desc = RADIAL_WORKLOADS[args.config]
    plan = tpc.Plan(irreps, lsh, lout, radial=radial, uvw=True)
    wl = make_workload(args.config, plan.dims(), seed=0)
    N, E = wl.n_nodes, wl.n_edges
    P, U = plan.n_paths, plan.mul
    NH = radial[1]
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    src, dst = T(wl.src), T(wl.dst)
    g = tpc.graph_build(src, dst, N)
    Y = tpc.sph_harm(lsh, tpc.gather_rows(T(wl.r), g.perm))
    rl = tpc.gather_rows(T(wl.r_len), g.perm)
    x, W1, W2, Wm, go = T(wl.x), T(wl.W1), T(wl.W2), T(wl.Wmix), T(wl.g)
    out = torch.empty(N, plan.outdim, device=dev)
    pre = torch.empty_like(out)
    outs = {"x": torch.empty_like(x), "Y": torch.empty_like(Y), "W1": torch.empty_like(W1),
            "W2": torch.empty_like(W2), "Wmix": torch.empty_like(Wm)}
    ws = torch.empty(tpc.radial_workspace(plan, N, True), dtype=torch.uint8, device=dev)
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB

    def step():
        tpc.forward_radial(plan, g, x, Y, rl, W1, W2, Wm, out=out, out_pre=pre)
        tpc.backward_radial(plan, g, x, Y, rl, W1, W2, go, Wmix=Wm, out_pre=pre, outs=outs, ws=ws)

    if args.counters:
        counters_run(torch, dev, flush, step, args.config)
        return
    do_flush, timed_steps, timed_kernel = make_timers(torch, flush)
    bwd = lambda want: (lambda: tpc.backward_radial(plan, g, x, Y, rl, W1, W2, go, want=want,
                                                    outs=outs, ws=ws))
    kernels = {
        "fwd": lambda: tpc.forward_radial(plan, g, x, Y, rl, W1, W2, None, out=pre),
        "bwd_recv": bwd(("Y", "W1")),
        "bwd_w2": bwd(("W2",)),
        "bwd_send": bwd(("x",)),
        "fwd_with_mix": lambda: tpc.forward_radial(plan, g, x, Y, rl, W1, W2, Wm, out=out,
                                                   out_pre=pre),
    }
    r_sorted = tpc.gather_rows(T(wl.r), g.perm)
    grl = torch.empty_like(rl)
    grad_r = torch.empty_like(r_sorted)
    outs_f = dict(outs, rlen=grl)
    extras = {
        # receiver pass that also returns the edge-length gradient, then the
        # edge-vector gradient
        "bwd_recv_with_rlen": lambda: tpc.backward_radial(plan, g, x, Y, rl, W1, W2, go,
                                                          want=("Y", "W1", "rlen"), outs=outs_f,
                                                          ws=ws),
        "forces": lambda: tpc.sph_harm_backward(lsh, r_sorted, outs["Y"], grl, out=grad_r),
    }
    flush.fill_(1.0)
    timed_steps(step, args.warmup, True)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    t = timed_steps(step, args.steps, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall0
    reps, rounds = 3, 2
    kt = {n: float(timed_kernel(fn, reps, rounds).mean()) for n, fn in kernels.items()}
    extra_ms = {n: float(timed_kernel(fn, reps, rounds).mean()) for n, fn in extras.items()}
    fl = radial_flops(E, P, U, NH)
    copy_gbs = copy_bandwidth(torch, dev, flush)
    wk = read_profile_value(args.config, "write_kib.fwd", RADIAL_SOURCES)
    fwd_write_ratio = None if wk is None else wk * 1024 / (4.0 * N * plan.outdim)
    names = ["fwd", "bwd_recv", "bwd_w2", "bwd_send"]
    dom = max(names, key=lambda n: kt[n])
    achieved = fl[dom] / (kt[dom] * 1e-3) / 1e12
    step_ms = float(t.mean())
    traffic = read_traffic(args.config, RADIAL_SOURCES)
    res = {
        "metric": METRIC,
        "value": E / (step_ms * 1e-3),
        "unit": "edges/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; random-init radial MLP and mix weights)",
        "config": {"workload": f"{args.config}: {desc}", "n_nodes": N, "n_edges": E,
                   "irreps": irreps, "lmax_sh": lsh, "lmax_out": lout, "paths": P,
                   "radial": {"basis": radial[0], "hidden": radial[1], "r_cut": radial[2]},
                   "mode": "fwd+bwd", "cache": "L2+MALL flushed before each step"},
        "fwd_edges_per_s": E / (kt["fwd_with_mix"] * 1e-3),
        "fwd_edges_per_s_note": "forward alone (radial pass + mix, launch durations)",
        "ms_per_step_p10_p90": [float(np.percentile(t, 10)), float(np.percentile(t, 90))],
        "kernel_ms": kt,
        "kernel_ms_note": f"per call, {reps} back-to-back calls after a cache flush, mean of "
                          f"{rounds}; bwd_recv and bwd_w2 include their partial-sum kernels",
        "kernel_mfma_frac": {n: fl[n] / (kt[n] * 1e-3) / 1e12 / FP32_MFMA_PEAK_TFLOPS
                             for n in names},
        "forces_ms": extra_ms,
        "forces_note": "receiver pass that also returns the edge-length gradient, and the "
                       "edge-vector gradient kernel; not part of the step",
        "copy_GBs": copy_gbs,
        "fwd_write_ratio": fwd_write_ratio,
        "fwd_write_note": "radial pass HBM writes (WRITE_SIZE, committed summary) over "
                          "N*outdim*4: no per-edge weight or message is written",
        "wall_s_timed_region": wall,
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": achieved,
                     "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / FP32_MFMA_PEAK_TFLOPS, "algorithmic_flops": fl[dom],
                     "traffic": (traffic or {}).get(dom)},
    }
    if not args.no_cpu_baseline:
        import oracle
        op = oracle.build_plan(irreps, lsh, lout)
        res["cpu_baseline"] = cpu_baseline_radial(op, wl, radial)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res))


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


def bench_fc(args, torch, tpc, make_workload, dev):
    from workloads import make_fc_inputs
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
    reps, rounds = 5, max(2, args.steps // 5)
    kt = {n: float(timed_kernel(fn, reps, rounds).mean()) for n, fn in phases.items()}
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
        "wall_s_timed_region": wall,
        "roofline": {"bound": "hbm", "kernel": f"{dom} (one entry-point call)",
                     "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes": alg[dom],
                     "note": "inputs and outputs once plus one write and one read of each "
                             "node-sized state the phase uses", "traffic": None},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        op = oracle.build_plan(irreps, lsh, lout)
        try:
            from threadpoolctl import threadpool_info
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        except Exception:
            threads = 1
        n_s = 12000
        order = np.argsort(wl.dst, kind="stable")[:n_s]
        e = np.sort(order)
        nodes = np.unique(np.concatenate([wl.src[e], wl.dst[e]]))
        src, dst = np.searchsorted(nodes, wl.src[e]), np.searchsorted(nodes, wl.dst[e])
        t0 = time.perf_counter()
        Yo = oracle.sh_real(lsh, wl.r[e])
        oracle.fc_conv_fwd(op, src, dst, len(nodes), wl.x[nodes], Yo, R[e], Th)
        oracle.fc_conv_bwd(op, src, dst, len(nodes), wl.x[nodes], Yo, R[e], Th, go_h[nodes])
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": len(e) / dt, "unit": "edges/s", "cores": int(threads),
                               "kind": "oracle",
                               "sample": f"{len(e)} of {E} edges (the first receivers), harmonics + "
                                         f"fwd + bwd once, float64 (per-edge weights formed), {dt:.2f} s"}
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


def bench_gaunt(args, torch, tpc, make_workload, dev):
    from workloads import make_gaunt_weights
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
    reps, rounds = 10, max(2, args.steps // 5)
    kt = {n: float(timed_kernel(fn, reps, rounds).mean()) for n, fn in kernels.items()}
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
    }
    if not args.no_cpu_baseline:
        import oracle
        try:
            from threadpoolctl import threadpool_info
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        except Exception:
            threads = 1
        gp = oracle.gaunt_plan(irreps, lsh, lout)
        dts = []
        for _ in range(3):
            t0 = time.perf_counter()
            Yo = oracle.sh_real(lsh, wl.r)
            oracle.gaunt_conv_fwd(gp, wl.src, wl.dst, N, wl.x, Yo, w)
            oracle.gaunt_conv_bwd(gp, wl.src, wl.dst, N, wl.x, Yo, w, go_h)
            dts.append(time.perf_counter() - t0)
        dt = float(np.median(dts))
        res["cpu_baseline"] = {"value": E / dt, "unit": "edges/s", "cores": int(threads),
                               "kind": "oracle",
                               "sample": f"the whole workload ({E} edges), harmonics + Gaunt fwd + bwd, "
                                         f"float64, median of 3 runs ({dt:.2f} s each)"}
    print(json.dumps(res))


if __name__ == "__main__":
    main()
