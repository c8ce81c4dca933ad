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
PROFILE_SUMMARY = os.path.join(ROOT, "profiles", "hbm_traffic_{}.txt")
KERNEL_SOURCES = ("conv_kernels.hpp", "sig.hpp", "cg_table.hpp")


def kernel_source_hash():
    h = hashlib.sha256()
    d = os.path.join(ROOT, "tensor_product_convolution_amd", "csrc")
    for f in KERNEL_SOURCES:
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
    }


def read_traffic(config):
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
    if vals.get("kernel_source_hash") != kernel_source_hash():
        return None          # kernels changed since the counters were taken
    out = {}
    for k, v in vals.items():
        if k.startswith("traffic_bytes."):
            out[k.split(".", 1)[1]] = float(v)
    return out or None


def cpu_baseline(op, wl):
    """The float64 oracle on this host, fwd + bwd over the whole workload."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = 1
    t0 = time.perf_counter()
    Y = oracle.sh_real(op.lmax_sh, wl.r)
    oracle.tp_conv_fwd(op, wl.src, wl.dst, wl.n_nodes, wl.x, Y, wl.w)
    oracle.tp_conv_bwd(op, wl.src, wl.dst, wl.n_nodes, wl.x, Y, wl.w, wl.g)
    dt = time.perf_counter() - t0
    return {"value": wl.n_edges / dt, "unit": "edges/s", "cores": int(threads), "kind": "oracle",
            "sample": f"whole workload ({wl.n_edges} edges), harmonics + fwd + bwd once, float64, "
                      f"{dt:.2f} s; host affinity {len(os.sched_getaffinity(0))} cores"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="mid", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--warm", action="store_true",
                    help="also time the steps back to back without the cache flush")
    ap.add_argument("--counters", action="store_true",
                    help="short run for rocprofv3 counter passes: a few steps plus a 512 MiB copy")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
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
    irreps, lsh, lout, desc = WORKLOADS[args.config]
    plan = tpc.Plan(irreps, lsh, lout)
    wl = make_workload(args.config, plan.dims(), seed=0)
    N, E = wl.n_nodes, wl.n_edges
    P, U, ysh = plan.n_paths, plan.mul, plan.ysh
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    src, dst = T(wl.src), T(wl.dst)
    g = tpc.graph_build(src, dst, N)
    Y = tpc.sph_harm(lsh, tpc.gather_rows(T(wl.r), g.perm))
    w = tpc.gather_rows(T(wl.w), g.perm)
    x, go = T(wl.x), T(wl.g)
    out = torch.empty(N, plan.outdim, device=dev)
    gx = torch.empty_like(x)
    gY = torch.empty_like(Y)
    gw = torch.empty_like(w)
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB

    def step():
        tpc.forward(plan, g, x, Y, w, out=out)
        tpc.backward(plan, g, x, Y, w, go, outs=(None, gY, gw))
        tpc.backward(plan, g, x, Y, w, go, outs=(gx, None, None))

    if args.counters:
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
        print(json.dumps({"counters_run": args.config, "copy_bytes": a.numel() * 4}))
        return

    def do_flush():
        # read 1 GiB: L2 and the Infinity Cache end up holding clean lines of
        # an unrelated buffer (a write would leave dirty lines whose write-back
        # competes with the next kernel's reads)
        flush.sum()

    def timed_steps(k, cold):
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

    kernels = {
        "fwd": lambda: tpc.forward(plan, g, x, Y, w, out=out),
        "bwd_recv": lambda: tpc.backward(plan, g, x, Y, w, go, outs=(None, gY, gw)),
        "bwd_send": lambda: tpc.backward(plan, g, x, Y, w, go, outs=(gx, None, None)),
    }

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

    names = ["fwd", "bwd_recv", "bwd_send"]
    kt = np.array([kt_all[n].mean() for n in names])     # ms per launch
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
                   "mode": "fwd+bwd", "cache": "L2+MALL flushed before each step"},
        "fwd_edges_per_s": E / (fwd_ms * 1e-3),
        "fwd_edges_per_s_note": "forward kernel alone (launch duration); value is the whole step",
        "ms_per_step_p10_p90": [float(np.percentile(t, 10)), float(np.percentile(t, 90))],
        "kernel_ms": {n: float(v) for n, v in zip(names, kt)},
        "kernel_ms_note": f"per launch, {reps} back-to-back launches after a cache flush, mean of {rounds}",
        "kernel_hbm_frac": {n: ab[n] / (float(v) * 1e-3) / 1e9 / HBM_PEAK_GBS for n, v in zip(names, kt)},
        "step_hbm_frac": ab["step"] / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
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
        res["cpu_baseline"] = cpu_baseline(op, wl)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res))


if __name__ == "__main__":
    main()
