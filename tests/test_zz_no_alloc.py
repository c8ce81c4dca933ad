"""The graph build that allocates nothing (tp_conv_graph_build_static, scratch in
a static device array of the library) against the build with a caller
workspace (tp_conv_graph_build): bit-identical arrays on consecutive calls,
the second with a smaller graph, so the scratch a call leaves behind cannot
leak into the next one.  Both calls go through the C ABI (ctypes)."""
import numpy as np
import pytest
import torch

import tensor_product_convolution_amd as tpc
from workloads import make_workload

pytestmark = pytest.mark.gpu

FIELDS = ("row_ptr", "col", "perm", "t_row_ptr", "t_perm", "t_col")


def _graph(name, n_nodes=None):
    wl = make_workload(name, {}, seed=0, n_nodes=n_nodes, graph_only=True)
    dev = torch.device("cuda:0")
    return (torch.from_numpy(wl.src).to(dev), torch.from_numpy(wl.dst).to(dev), wl.n_nodes)


def _same(a, b):
    for f in FIELDS:
        x, y = getattr(a, f), getattr(b, f)
        assert x.shape == y.shape and torch.equal(x, y), f


def test_static_build_matches_workspace_build_on_consecutive_calls():
    cases = [("zipf", 8192), ("mid", None), ("tiny", None), ("lmax3", 600)]   # sizes fall, then rise
    for name, n in cases:
        src, dst, N = _graph(name, n)
        print(f"static graph build: {name} N={N} E={src.shape[0]}", flush=True)
        ref = tpc.graph_build(src, dst, N)
        got = tpc.graph_build_static(src, dst, N)
        torch.cuda.synchronize()
        _same(got, ref)
        # the unchecked build too (no host synchronisation inside the call)
        got2 = tpc.graph_build_static(src, dst, N, check=False)
        torch.cuda.synchronize()
        _same(got2, ref)


def test_static_build_fills_given_arrays_and_handles_empty_and_isolated_nodes():
    dev = torch.device("cuda:0")
    src, dst, N = _graph("mid")
    ref = tpc.graph_build(src, dst, N)
    out = tpc.graph_build_static(src, dst, N)
    # refill the same arrays from a smaller graph of the same sizes: a permutation
    # of the edge list changes every array
    rng = np.random.default_rng(5)
    p = torch.from_numpy(rng.permutation(src.shape[0]).astype(np.int64)).to(dev)
    ref2 = tpc.graph_build(src[p].contiguous(), dst[p].contiguous(), N)
    got2 = tpc.graph_build_static(src[p].contiguous(), dst[p].contiguous(), N, out=out)
    torch.cuda.synchronize()
    assert got2 is out
    _same(got2, ref2)
    # no edges at all, and nodes without edges
    e0 = torch.zeros(0, dtype=torch.int32, device=dev)
    z = tpc.graph_build_static(e0, e0, 5)
    torch.cuda.synchronize()
    assert z.row_ptr.tolist() == [0] * 6 and z.t_row_ptr.tolist() == [0] * 6
    s1 = torch.tensor([3, 3, 0], dtype=torch.int32, device=dev)
    d1 = torch.tensor([1, 1, 3], dtype=torch.int32, device=dev)
    _same(tpc.graph_build_static(s1, d1, 6), tpc.graph_build(s1, d1, 6))


def test_static_build_rejects_a_graph_beyond_its_scratch():
    dev = torch.device("cuda:0")
    E = 2_000_000
    src = torch.zeros(E, dtype=torch.int32, device=dev)
    with pytest.raises(tpc.TPError) as e:
        tpc.graph_build_static(src, src, 10)
    assert "static scratch" in str(e.value)
