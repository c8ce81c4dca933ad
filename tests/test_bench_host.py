"""Host-side logic of bench.py (no GPU): the one-GPU guard, the algorithmic
byte and flop counts the roofline lines divide by, the cold-copy count, the
pooled CPU baseline, and the reading of the committed counter summaries."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_of_the_1536_atom_workload():
    # 46,080 edges, 15 paths x 32 channels, 9 harmonics; x 288 and out 544 floats per node
    ab = bench.algorithmic_bytes(1536, 46080, 15, 32, 9, 288, 544)
    per_node = 4 * 1536 * (288 + 544 + 1)
    assert ab["fwd"] == 46080 * (4 * 480 + 36 + 4) + per_node          # w, Y, col once; x, out, row_ptr
    assert ab["bwd_recv"] == 46080 * (8 * 480 + 72 + 4) + per_node     # grad_w and grad_Y written too
    assert ab["bwd_send"] == 46080 * (4 * 480 + 36 + 8) + per_node     # t_perm and t_col
    # one-pass backward: w, Y, t_perm, t_col in; grad_w, grad_Y out; x, grad_out, t_row_ptr in; grad_x out
    assert ab["bwd"] == 46080 * (8 * 480 + 72 + 8) + 4 * 1536 * (2 * 288 + 544 + 1)
    assert ab["step"] == 46080 * (8 * 480 + 72 + 4) + 4 * 1536 * (2 * 288 + 2 * 544 + 1)
    assert round(ab["fwd"] / 1e6, 1) == 95.4 and round(ab["bwd_recv"] / 1e6, 1) == 185.6
    assert round(ab["step"] / 1e6, 1) == 190.7
    # forward + backward, each pass touching its arrays once: 282.96 MB
    assert round(bench.step_bytes(ab, False) / 1e6, 2) == 282.96
    assert bench.step_bytes(ab, True) == ab["fwd"]
    # second-order backward: three edge streams in (w, gg_w; Y, gg_Y), one out
    # (d_w; d_Y), three index arrays; x, gg_x, d_x, grad_out, d_grad_out, two row pointers
    assert ab["double_bwd"] == 46080 * (12 * 480 + 108 + 12) + 4 * 1536 * (3 * 288 + 2 * 544 + 2)
    assert round(ab["double_bwd"] / 1e6, 1) == 283.0


def test_algorithmic_bytes_of_the_edge_vector_form():
    # r (12 B) replaces Y (36 B) in, grad_r (12 B) replaces grad_Y (36 B) out
    ab = bench.algorithmic_bytes_geom(1536, 46080, 15, 32, 288, 544)
    assert ab["fwd_r"] == 46080 * (4 * 480 + 12 + 4) + 4 * 1536 * (288 + 544 + 1)
    assert ab["bwd_r"] == 46080 * (8 * 480 + 24 + 8) + 4 * 1536 * (2 * 288 + 544 + 1)
    y = bench.algorithmic_bytes(1536, 46080, 15, 32, 9, 288, 544)
    assert y["fwd"] - ab["fwd_r"] == 46080 * 24 and y["bwd"] - ab["bwd_r"] == 46080 * 48


def _oracle_counts(irreps, lsh):
    """the same counts taken from the oracle's dense tables (independent of the
    library's plan and of bench.cg_counts)"""
    import oracle
    op = oracle.build_plan(irreps, lsh, lsh)
    nnz, ab, gc, d2, d3 = 0, set(), set(), 0, 0
    for (i, l1, l2, l3, k), C in zip(op.paths, op.cg):
        C = np.asarray(C)
        d2 += 2 * l2 + 1
        d3 += 2 * l3 + 1
        for a, b, c in np.argwhere(np.abs(C) > 1e-12):
            nnz += 1
            ab.add((l1, l2, a, b))
            m = float(np.float32(abs(C[a, b, c])))
            if m != 1.0:
                gc.add((k, c, m))
    return {"nnz": nnz, "ab": len(ab), "d2": d2, "d3": d3, "gc": len(gc)}


@pytest.mark.parametrize("irreps,lsh", [("8x0e+8x1o", 2), ("32x0e+32x1o+32x2e", 2),
                                        ("64x0e+64x1o+64x2e+64x3o", 3)])
def test_cg_operation_counts(irreps, lsh):
    import tensor_product_convolution_amd as tpc
    plan = tpc.Plan(irreps, lsh, lsh)
    cnt = bench.cg_counts(plan.paths(), *plan.cg())
    assert cnt == _oracle_counts(irreps, lsh)
    fl = bench.cg_flops(cnt)
    if irreps.startswith("32x"):
        assert cnt == {"nnz": 137, "ab": 81, "d2": 51, "d3": 51, "gc": 42}
        assert fl["fwd"] == 81 + 2 * 137 + 2 * 51 and fl["bwd"] == 42 + 4 * 137 + 4 * 51 + 2 * 81


def test_radial_flops():
    # 3,000,000 edges, 15 paths x 128 channels, 64 hidden units: one [E x 64] x
    # [64 x 1920] product is 0.737 TFLOP; the second-order backward forms ten
    fl = bench.radial_flops(3_000_000, 15, 128, 64)
    assert round(fl["fwd"] / 1e12, 3) == 0.737
    assert fl["bwd_recv"] == 2 * fl["fwd"] and fl["double_bwd"] == 10 * fl["fwd"]


def test_cold_copy_count():
    assert bench.copies_for_cold(90e6) == 12            # 1,536-atom w + Y: 12 x 90 MB >= 1 GiB
    assert bench.copies_for_cold(7e9) == 1              # the Zipf weight stream alone is cold
    assert bench.copies_for_cold(1) == 16               # capped


def test_receiver_split_keeps_receivers_whole():
    rng = np.random.default_rng(3)
    dst = rng.integers(0, 50, size=1000)
    chunks = bench._chunks_by_receiver(dst, 7)
    allc = np.concatenate(chunks)
    assert sorted(allc.tolist()) == list(range(1000))
    owners = {}
    for t, c in enumerate(chunks):
        for i in np.unique(dst[c]):
            assert owners.setdefault(int(i), t) == t       # no receiver in two chunks


def test_pooled_oracle_equals_one_process():
    """The CPU baseline's pooled evaluation sums the same results as one call."""
    import oracle
    from workloads import make_workload
    op = oracle.build_plan("8x0e+8x1o", 2, 2)
    dims = dict(xdim=op.xdim, n_paths=op.n_paths, U=op.U, outdim=op.outdim, n_out_irreps=5)
    wl = make_workload("tiny", dims, seed=0)
    (out, gx, gY, gw), dt = bench.pooled_oracle_direct(("8x0e+8x1o", 2, 2), wl.src, wl.dst, wl.n_nodes,
                                                       wl.x, wl.r, wl.w, wl.g, 3)
    Y = oracle.sh_real(2, wl.r)
    ref = oracle.tp_conv_fwd(op, wl.src, wl.dst, wl.n_nodes, wl.x, Y, wl.w)
    rx, rY, rw = oracle.tp_conv_bwd(op, wl.src, wl.dst, wl.n_nodes, wl.x, Y, wl.w, wl.g)
    for got, want in ((out, ref), (gx, rx), (gY, rY), (gw, rw)):
        assert np.allclose(got, want, rtol=1e-12, atol=1e-12)
    assert dt > 0


def test_fc_and_gaunt_counts():
    d3 = [1, 3, 5, 3, 1, 3, 5, 3, 5, 5, 3, 5, 1, 3, 5]                    # sum 51
    d1 = [1, 1, 1, 3, 3, 3, 3, 3, 3, 5, 5, 5, 5, 5, 5]
    fc = bench.fc_algorithmic(1536, 46080, 15, 32, 8, d3, d1, 288, 544, 9)
    s_state = 4.0 * 1536 * 8 * 32 * 51
    assert fc["fwd"] > 2 * s_state and fc["bwd_theta"] > s_state
    assert fc["bwd_theta"] == 4.0 * 1536 * 544 + 4.0 * 8 * 15 * 32 * 32 + s_state
    ga = bench.gaunt_algorithmic(1536, 46080, 32, 288, 9, 96, 288)
    for k in ("fwd", "bwd_recv", "bwd_send"):
        assert ga[k]["flops"] > 0 and ga[k]["bytes"] > 0


@pytest.mark.parametrize("config,sources", [("mid", bench.KERNEL_SOURCES), ("fc", bench.FC_SOURCES),
                                            ("gaunt", bench.GAUNT_SOURCES),
                                            ("stream", bench.RADIAL_SOURCES["stream"]),
                                            ("lmax3_radial", bench.RADIAL_SOURCES["lmax3_radial"])])
def test_counter_summaries_parse(config, sources):
    # null once the kernel sources change after the counters were taken, else
    # one positive byte count per kernel of the step
    t = bench.read_traffic(config, sources)
    assert t is None or (len(t) >= 2 and all(v > 0 for v in t.values()))


def _direct_snapshot(op, wl):
    """what the timed step leaves on the GPU, here from the oracle in float32:
    out, grad_x, and receiver-sorted grad_Y / grad_w with the permutation"""
    import oracle
    Y = oracle.sh_real(op.lmax_sh, wl.r)
    ref = oracle.tp_conv_fwd(op, wl.src, wl.dst, wl.n_nodes, wl.x, Y, wl.w)
    rx, rY, rw = oracle.tp_conv_bwd(op, wl.src, wl.dst, wl.n_nodes, wl.x, Y, wl.w, wl.g)
    perm = oracle.csr_build(wl.src, wl.dst, wl.n_nodes)["perm"]
    f = lambda a: a.astype(np.float32)
    return dict(out=f(ref), gx=f(rx), gY=f(rY[perm]), gw=f(rw[perm]), perm=perm)


@pytest.mark.parametrize("max_edges", [100000, 300])
def test_parity_on_the_cpu_baseline_sample(max_edges):
    """The bench line's parity entry: the timed step's outputs against the
    oracle on the CPU-baseline sample (whole workload, or the edges into the
    first receivers); float32 copies of the oracle's own results pass, and an
    error planted in one path block of one sampled edge is reported."""
    import oracle
    from workloads import make_workload
    irr = "8x0e+8x1o+8x2e"
    op = oracle.build_plan(irr, 2, 2)
    dims = dict(xdim=op.xdim, n_paths=op.n_paths, U=op.U, outdim=op.outdim, n_out_irreps=5)
    wl = make_workload("mid", dims, seed=2, n_nodes=40)
    snap = _direct_snapshot(op, wl)
    bench.cpu_baseline_direct(irr, 2, 2, wl, False, max_edges, snap=snap)
    par = snap["parity"]
    assert par["max_rel_err"] < 1e-6
    assert set(par["per_output"]) == ({"out", "grad_Y", "grad_w", "grad_x"} if max_edges > wl.n_edges
                                      else {"out", "grad_Y", "grad_w"})
    # plant: the first sampled edge (the first receiver's first edge) at its sorted position 0
    bad = _direct_snapshot(op, wl)
    bad["gw"][0, 3, :] += 0.01 * np.max(np.abs(bad["gw"][:, 3, :]))
    bench.cpu_baseline_direct(irr, 2, 2, wl, False, max_edges, snap=bad)
    assert bad["parity"]["per_output"]["grad_w"] > 1e-3
    assert bad["parity"]["per_output"]["out"] < 1e-6


def test_parity_of_the_radial_sample():
    """The same for the radial layer: the mixed output of the sampled
    receivers and grad_Y of their edges."""
    import oracle
    from workloads import make_workload
    irr = "4x0e+4x1o+4x2e"
    op = oracle.build_plan(irr, 2, 2)
    dims = dict(xdim=op.xdim, n_paths=op.n_paths, U=op.U, outdim=op.outdim, n_out_irreps=5)
    wl = make_workload("stream", dims, seed=3, n_nodes=50)
    Y = oracle.sh_real(2, wl.r)
    out = oracle.tp_conv_radial_fwd(op, wl.src, wl.dst, wl.n_nodes, wl.x, Y, wl.r_len, wl.W1, wl.W2,
                                    wl.Wmix, 8, 5.0)
    gY = oracle.tp_conv_radial_bwd(op, wl.src, wl.dst, wl.n_nodes, wl.x, Y, wl.r_len, wl.W1, wl.W2,
                                   wl.Wmix, wl.g, 8, 5.0)[1]
    perm = oracle.csr_build(wl.src, wl.dst, wl.n_nodes)["perm"]
    snap = dict(out=out.astype(np.float32), gY=gY[perm].astype(np.float32), perm=perm)
    bench.cpu_baseline_radial(irr, 2, 2, wl, (8, 64, 5.0), max_edges=400, snap=snap)
    assert snap["parity"]["max_rel_err"] < 1e-6
    snap["gY"][0, 5] += 0.01 * np.max(np.abs(snap["gY"][:, 4:9]))
    bench.cpu_baseline_radial(irr, 2, 2, wl, (8, 64, 5.0), max_edges=400, snap=snap)
    assert snap["parity"]["per_output"]["grad_Y"] > 1e-3


def test_sender_layout_bytes_and_node_order_copy():
    """The sender-grouped layout moves the same bytes over a step (the forward
    reads e_pos, the backward no t_perm), and the node-order copy of a graph
    drops only the launch orders."""
    ab = bench.algorithmic_bytes(1536, 46080, 15, 32, 9, 288, 544)
    assert ab["fwd_sg"] == ab["fwd"] + 4 * 46080
    assert ab["bwd_sg"] == ab["bwd"] - 4 * 46080
    assert ab["fwd_sg"] + ab["bwd_sg"] == ab["fwd"] + ab["bwd"]

    class G:
        pass
    g = G()
    g.row_ptr, g.order, g.t_order = object(), object(), object()
    h = bench.node_order(g)
    assert h.order is None and h.t_order is None and h.row_ptr is g.row_ptr
    assert g.order is not None and g.t_order is not None
