"""Host-side logic of bench.py (no GPU): the one-GPU guard, the algorithmic
byte and flop counts the roofline lines divide by, and the reading of the
committed counter summaries."""
import os
import subprocess
import sys

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
    assert ab["step"] == 46080 * (8 * 480 + 72 + 4) + 4 * 1536 * (2 * 288 + 2 * 544 + 1)
    assert round(ab["fwd"] / 1e6, 1) == 95.4 and round(ab["bwd_recv"] / 1e6, 1) == 185.6
    assert round(ab["step"] / 1e6, 1) == 190.7
    # second-order backward: three edge streams in (w, gg_w; Y, gg_Y), one out
    # (d_w; d_Y), three index arrays; x, gg_x, d_x, grad_out, d_grad_out, two row pointers
    assert ab["double_bwd"] == 46080 * (12 * 480 + 108 + 12) + 4 * 1536 * (3 * 288 + 2 * 544 + 2)
    assert round(ab["double_bwd"] / 1e6, 1) == 283.0


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
                                            ("gaunt", bench.GAUNT_SOURCES)])
def test_counter_summaries_parse(config, sources):
    # null once the kernel sources change after the counters were taken, else
    # one positive byte count per kernel of the step
    t = bench.read_traffic(config, sources)
    assert t is None or (len(t) >= 3 and all(v > 0 for v in t.values()))
