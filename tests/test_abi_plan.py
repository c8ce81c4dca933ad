"""The C ABI library loads, exports every declared symbol, builds the same
plan tables as the oracle and rejects bad arguments before any launch.

These run on the CPU: plan calls are host-only, and every error case below is
caught by host validation before a HIP call is made.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import tensor_product_convolution_amd as tpc

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "tpconv.h")

pytestmark = pytest.mark.skipif(not os.path.exists(tpc.LIB_PATH),
                                reason="libtpconv.so not built (run __graft_entry__.build())")


def test_library_exports_every_declared_symbol():
    src = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:tp_status|void|const char\*)\s+(\w+)\s*\(", src, re.M))
    assert declared == set(tpc.EXPORTS)
    L = ctypes.CDLL(tpc.LIB_PATH)
    for name in declared:
        assert hasattr(L, name), name


CONFIGS = [("8x0e+8x1o", 2, 2), ("32x0e+32x1o+32x2e", 2, 2),
           ("64x0e+64x1o+64x2e+64x3o", 3, 3), ("128x0e+128x1o+128x2e", 2, 2),
           ("16x0e+16x1o", 2, 2), ("64x0e+64x1o+64x2e", 2, 2)]


@pytest.mark.parametrize("irreps,lsh,lout", CONFIGS)
def test_plan_matches_oracle(irreps, lsh, lout):
    p = tpc.Plan(irreps, lsh, lout)
    o = oracle.build_plan(irreps, lsh, lout)
    assert (p.n_paths, p.mul, p.xdim, p.ysh, p.outdim, p.nnz) == (
        o.n_paths, o.U, o.xdim, o.ysh, o.outdim, o.nnz())
    assert p.out_irreps == o.out_irreps_str()
    assert p.paths() == [(l1, l2, l3, k) for _, l1, l2, l3, k in o.paths]
    idx, val = p.cg()
    want_idx, want_val = [], []
    for q, C in enumerate(o.cg):
        for a, b, c in np.argwhere(C != 0):
            want_idx.append((q, a, b, c))
            want_val.append(C[a, b, c])
    assert np.array_equal(idx.astype(np.int64), np.array(want_idx, dtype=np.int64))
    assert np.max(np.abs(val - np.array(want_val))) <= 1e-12


def test_dense_cg_builder_matches_oracle_up_to_l4():
    for l1 in range(5):
        for l2 in range(5):
            for l3 in range(5):
                got = tpc.cg_real(l1, l2, l3)
                want = oracle.cg_real(l1, l2, l3)
                assert np.max(np.abs(got - want)) <= 1e-12, (l1, l2, l3)


def _status(fn, *args):
    return fn(*args)


def test_plan_errors():
    L = tpc.lib()
    h = ctypes.c_void_p()
    cases = [("8x0e+4x1o", 2, 2, -2), ("8x1e", 2, 2, -2), ("8x0q", 2, 2, -2), ("", 2, 2, -2),
             ("8x0e+8x1o+8x2e+8x3o+8x4e", 2, 2, -3), ("8x0e+8x1o", 5, 5, -3),
             ("12x0e+12x1o", 2, 2, -3), ("8x0e", -1, 2, -1)]
    for irr, ls, lo, want in cases:
        st = L.tp_conv_plan_create(ctypes.byref(h), irr.encode(), ls, lo, 0, None)
        assert st == want, (irr, st, L.tp_conv_last_error())
        assert not h.value
    assert L.tp_conv_plan_create(None, b"8x0e", 0, 0, 0, None) == -1
    assert L.tp_conv_plan_create(ctypes.byref(h), b"8x0e+8x1o", 2, 2, 7, None) == -3
    with pytest.raises(tpc.TPError) as e:
        tpc.Plan("8x0e+8x1e", 2, 2)
    assert "natural parity" in str(e.value)
    assert L.tp_cg_real(7, 0, 7, None) == -1


def test_graph_and_conv_argument_errors_without_launch():
    L = tpc.lib()
    p = tpc.Plan("8x0e+8x1o", 2, 2)
    assert L.tp_conv_forward(p.handle, None, None, None, None, None, None) == -1
    g = tpc._Graph(4, 10, None, None, None, None, None, None)
    assert L.tp_conv_forward(p.handle, ctypes.byref(g), None, None, None, None, None) == -1
    assert L.tp_conv_forward(None, ctypes.byref(g), None, None, None, None, None) == -1
    g2 = tpc._Graph(-1, 0, None, None, None, None, None, None)
    assert L.tp_conv_backward(p.handle, ctypes.byref(g2), None, None, None, None, None, None,
                              None, None) == -1
    need = ctypes.c_size_t()
    assert L.tp_conv_graph_workspace(100, 1000, ctypes.byref(need)) == 0 and need.value > 4000
    assert L.tp_conv_graph_workspace(-1, 10, ctypes.byref(need)) == -1
    fake = ctypes.c_void_p(0x1000)
    # workspace too small is reported before any launch
    assert L.tp_conv_graph_build(fake, fake, 1000, 100, fake, fake, fake, fake, fake, fake, fake, 16,
                                 0, None) == -5
    assert L.tp_conv_graph_build(None, None, 1000, 100, fake, fake, fake, fake, fake, fake, fake,
                                 need.value, 0, None) == -1
    assert L.tp_conv_graph_build(fake, fake, 10, 0, fake, fake, fake, fake, fake, fake, fake,
                                 need.value, 0, None) == -1
    assert L.tp_conv_sph_harm(2, None, 5, None, None) == -1
    assert L.tp_conv_gather_rows(None, None, 5, 3, None, None) == -1
    assert L.tp_conv_gather_rows(fake, fake, -1, 3, fake, None) == -1
    msg = L.tp_conv_last_error().decode()
    assert "negative" in msg
