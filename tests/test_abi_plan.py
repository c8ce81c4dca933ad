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
           ("16x0e+16x1o", 2, 2), ("64x0e+64x1o+64x2e", 2, 2),
           ("32x0e+32x1o", 1, 1), ("64x0e+64x1o", 3, 3)]


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
    # the graph build without a workspace: argument errors and a graph beyond its
    # static scratch are reported before any HIP call
    assert L.tp_conv_graph_build_static(fake, fake, 10, 0, fake, fake, fake, fake, fake, fake, 0, None) == -1
    assert L.tp_conv_graph_build_static(None, None, 10, 4, fake, fake, fake, fake, fake, fake, 0, None) == -1
    big = 2_000_000
    assert L.tp_conv_graph_workspace(100000, big, ctypes.byref(need)) == 0 and need.value > 24 << 20
    assert L.tp_conv_graph_build_static(fake, fake, big, 100000, fake, fake, fake, fake, fake, fake, 0,
                                        None) == -5
    assert "static scratch" in L.tp_conv_last_error().decode()
    assert L.tp_conv_sph_harm(2, None, 5, None, None) == -1
    assert L.tp_conv_gather_rows(None, None, 5, 3, None, None) == -1
    assert L.tp_conv_gather_rows(fake, fake, -1, 3, fake, None) == -1
    msg = L.tp_conv_last_error().decode()
    assert "negative" in msg
    # more rows than the int32 edge indices can address
    assert L.tp_conv_gather_rows(fake, fake, 1 << 31, 3, fake, None) == -4


def test_conv_alignment_errors_without_launch():
    """Rows of x, w and grad_out are staged with 16-byte loads: a pointer that is
    only 4-byte aligned is rejected on the host (no launch), for the forward,
    the backward and the channel mix."""
    L = tpc.lib()
    p = tpc.Plan("8x0e+8x1o", 2, 2)
    mix = tpc.Plan("16x0e+16x1o+16x2e", 2, 2, uvw=True)
    fake, odd = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x1004)
    out = ctypes.c_void_p(0x3000)
    g = tpc._Graph(4, 10, fake, fake, fake, fake, fake, fake)
    assert L.tp_conv_forward(p.handle, ctypes.byref(g), odd, fake, fake, out, None) == -1
    assert "16-byte" in L.tp_conv_last_error().decode()
    assert L.tp_conv_forward(p.handle, ctypes.byref(g), fake, fake, odd, out, None) == -1
    # x, Y, w, grad_out | grad_x, grad_Y, grad_w
    for bad in range(4):
        args = [fake] * 4
        if bad != 1:                     # Y rows move as 4-byte granules
            args[bad] = odd
            assert L.tp_conv_backward(p.handle, ctypes.byref(g), *args, out, out, out, None) == -1
            assert "16-byte" in L.tp_conv_last_error().decode()
    assert L.tp_conv_uvw_forward(mix.handle, 4, fake, fake, odd, None) == -1
    assert L.tp_conv_uvw_backward(mix.handle, 4, fake, odd, fake, out, None, fake, 1 << 30, None) == -1
    assert L.tp_conv_uvw_backward(mix.handle, 4, fake, fake, odd, out, None, fake, 1 << 30, None) == -1
    assert "16-byte" in L.tp_conv_last_error().decode()
    L.tp_conv_plan_destroy(None)          # NULL is ignored


def test_radial_uvw_forces_double_argument_errors_without_launch():
    """Host validation of the radial, mix, forces and second-order entry points:
    every case returns its status before any HIP call."""
    L = tpc.lib()
    fake = ctypes.c_void_p(0x1000)
    odd = ctypes.c_void_p(0x1004)                  # not 16-byte aligned
    plain = tpc.Plan("16x0e+16x1o+16x2e", 2, 2)
    rad = tpc.Plan("16x0e+16x1o+16x2e", 2, 2, radial=(8, 64, 5.0), uvw=True)
    g = tpc._Graph(4, 10, fake, fake, fake, fake, fake, fake)
    sz = ctypes.c_size_t()
    # radial workspace: only for radial plans; a mix adds to it
    assert L.tp_conv_radial_workspace(plain.handle, 4, 0, ctypes.byref(sz)) == -3
    assert L.tp_conv_radial_workspace(rad.handle, -1, 0, ctypes.byref(sz)) == -1
    assert L.tp_conv_radial_workspace(rad.handle, 4, 0, ctypes.byref(sz)) == 0 and sz.value > 0
    base = sz.value
    assert L.tp_conv_radial_workspace(rad.handle, 4, 1, ctypes.byref(sz)) == 0 and sz.value > base
    # radial forward / backward
    assert L.tp_conv_forward_radial(plain.handle, ctypes.byref(g), fake, fake, fake, fake, fake, None,
                                    None, fake, None) == -3
    assert L.tp_conv_forward_radial(rad.handle, ctypes.byref(g), fake, fake, fake, fake, fake, fake,
                                    fake, fake, None) == -1          # out_pre aliases out
    # x, Y, r_len, W1, W2 | Wmix, out_pre | grad_out | grad_x, grad_Y, grad_rlen, grad_W1, grad_W2 | grad_Wmix
    args = [fake] * 5 + [None, None] + [fake] + [fake] * 5 + [None]
    assert L.tp_conv_backward_radial(None, ctypes.byref(g), *args, fake, 1 << 30, None) == -1
    assert L.tp_conv_backward_radial(plain.handle, ctypes.byref(g), *args, fake, 1 << 30, None) == -3
    assert L.tp_conv_backward_radial(rad.handle, ctypes.byref(g), *args, fake, 16, None) == -5
    bad = [odd] + [fake] * 4 + [None, None] + [fake] + [fake] * 5 + [None]
    assert L.tp_conv_backward_radial(rad.handle, ctypes.byref(g), *bad, fake, 1 << 30, None) == -1
    assert "aligned" in L.tp_conv_last_error().decode()
    nomix = [fake] * 5 + [None, None] + [fake] + [fake] * 5 + [fake]   # grad_Wmix without Wmix
    assert L.tp_conv_backward_radial(rad.handle, ctypes.byref(g), *nomix, fake, 1 << 30, None) == -1
    # mix
    assert L.tp_conv_uvw_forward(rad.handle, 4, fake, fake, fake, None) == -1      # in == out
    assert L.tp_conv_uvw_forward(rad.handle, -1, fake, fake, ctypes.c_void_p(0x2000), None) == -1
    assert L.tp_conv_uvw_forward(rad.handle, 4, fake, odd, ctypes.c_void_p(0x2000), None) == -1
    assert L.tp_conv_uvw_backward(rad.handle, 4, fake, fake, fake, None, fake, fake, 16, None) == -5
    # forces
    assert L.tp_conv_sph_harm_backward(2, None, 5, fake, None, fake, None) == -1
    assert L.tp_conv_sph_harm_backward(2, fake, -1, fake, None, fake, None) == -1
    assert L.tp_conv_sph_harm_backward(4, fake, 5, fake, None, fake, None) == -3
    # second order
    assert L.tp_conv_double_backward(None, ctypes.byref(g), *([fake] * 4), None, None, None,
                                     fake, fake, fake, fake, None) == -1
    assert L.tp_conv_double_backward(plain.handle, None, *([fake] * 4), None, None, None,
                                     fake, fake, fake, fake, None) == -1
    assert L.tp_conv_double_backward(plain.handle, ctypes.byref(g), None, fake, fake, fake, None, None,
                                     None, fake, fake, fake, fake, None) == -1
    # plan options
    h = ctypes.c_void_p()
    o = tpc._Opts(8, 0, 5.0, 0)
    assert L.tp_conv_plan_create(ctypes.byref(h), b"16x0e+16x1o+16x2e", 2, 2, 0, ctypes.byref(o)) == -1
    o = tpc._Opts(8, 64, 5.0, 0)
    assert L.tp_conv_plan_create(ctypes.byref(h), b"16x0e+16x1o", 2, 2, 0, ctypes.byref(o)) == -3
    o = tpc._Opts(0, 0, 0.0, 1)
    assert L.tp_conv_plan_create(ctypes.byref(h), b"24x0e+24x1o", 2, 2, 0, ctypes.byref(o)) == -3


def test_fc_and_gaunt_host_validation_without_launch():
    """Sizes and host validation of the fully connected and Gaunt entry points;
    every error case returns before any HIP call."""
    L = tpc.lib()
    G = tpc.TP_MODE_GAUNT
    fake = ctypes.c_void_p(0x1000)
    odd = ctypes.c_void_p(0x1004)
    g = tpc._Graph(4, 10, fake, fake, fake, fake, fake, fake)
    sz = ctypes.c_size_t()
    p = tpc.Plan("32x0e+32x1o+32x2e", 2, 2, mode=G)
    # Gaunt plan: even couplings only, outputs 0e+1o+2e, no CG table
    o = oracle.gaunt_plan("32x0e+32x1o+32x2e", 2, 2)
    assert sorted(t[0:3] for t in p.paths()) == sorted(o.G)
    assert p.out_irreps == o.out_irreps_str() and p.outdim == o.outdim and p.nnz == 0
    # sizes: outdim U (lmax_out+1)^2, weights U (lmax_sh+1), a 32-point grid
    assert tpc.gaunt_dims(p) == (32 * 9, 32 * 3, 32)
    assert tpc.gaunt_dims(tpc.Plan("16x1o+16x0e", 1, 2, mode=G)) == (16 * 9, 16 * 2, 32)
    assert tpc.gaunt_dims(tpc.Plan("64x2e", 1, 1, mode=G)) == (64 * 4, 64 * 2, 32)
    h = ctypes.c_void_p()
    for irr, lsh, lout in (("8x0e+8x1o", 2, 2), ("64x0e+64x1o+64x2e+64x3o", 3, 3),
                           ("16x0e+16x1o", 3, 2), ("16x1o+16x1o", 2, 2)):
        assert L.tp_conv_plan_create(ctypes.byref(h), irr.encode(), lsh, lout, G, None) == -3
        assert not h.value
    assert L.tp_conv_plan_create(ctypes.byref(h), b"16x2e", 0, 1, G, None) == -1   # no even coupling
    # the CG entry points reject a Gaunt plan; the Gaunt ones reject a CG plan
    cg = tpc.Plan("32x0e+32x1o+32x2e", 2, 2)
    assert L.tp_conv_forward(p.handle, ctypes.byref(g), fake, fake, fake, fake, None) == -3
    assert L.tp_conv_forward_gaunt(cg.handle, ctypes.byref(g), fake, fake, fake, fake, None) == -3
    dims = [ctypes.c_int32() for _ in range(3)]
    assert L.tp_conv_gaunt_dims(cg.handle, *[ctypes.byref(d) for d in dims]) == -3
    assert L.tp_conv_fc_workspace(p.handle, 10, 8, ctypes.byref(sz)) == -3
    assert L.tp_conv_forward_gaunt(p.handle, ctypes.byref(g), fake, None, fake, fake, None) == -1
    assert L.tp_conv_forward_gaunt(p.handle, ctypes.byref(g), fake, fake, fake, None, None) == -1
    assert L.tp_conv_forward_gaunt(p.handle, None, fake, fake, fake, fake, None) == -1
    # Gaunt backward: plan mode, the sender grouping for grad_x, grad_out, w alignment
    gg = tpc._Graph(4, 10, fake, fake, fake, None, None, None)
    assert L.tp_conv_backward_gaunt(cg.handle, ctypes.byref(g), fake, fake, fake, fake, fake, fake, fake,
                                    None) == -3
    assert L.tp_conv_backward_gaunt(p.handle, ctypes.byref(gg), fake, fake, fake, fake, fake, None, None,
                                    None) == -1                                      # no t_row_ptr
    assert L.tp_conv_backward_gaunt(p.handle, ctypes.byref(g), fake, fake, fake, None, None, fake, fake,
                                    None) == -1                                      # no grad_out
    assert L.tp_conv_backward_gaunt(p.handle, ctypes.byref(g), fake, fake, odd, fake, None, fake, fake,
                                    None) == -1
    assert "aligned" in L.tp_conv_last_error().decode()
    # fully connected: sizes, unsupported shapes, workspace and alignment
    assert L.tp_conv_fc_workspace(cg.handle, 10, 8, ctypes.byref(sz)) == 0 and sz.value > 0
    assert L.tp_conv_fc_workspace(cg.handle, 10, 4, ctypes.byref(sz)) == -3
    assert L.tp_conv_forward_fc(cg.handle, ctypes.byref(g), fake, fake, fake, 8, fake, fake, fake,
                                16, None) == -5
    assert L.tp_conv_forward_fc(cg.handle, ctypes.byref(g), fake, fake, fake, 8, fake, fake, odd,
                                1 << 30, None) == -1
    # fully connected backward: flags, workspace, alignment, the sender grouping for grad_x
    assert L.tp_conv_fc_backward_workspace(cg.handle, 4, 8, ctypes.byref(sz)) == 0   # g has 4 nodes
    need = sz.value
    assert L.tp_conv_fc_workspace(cg.handle, 4, 8, ctypes.byref(sz)) == 0 and need > sz.value
    args = (fake, fake, fake, 8, fake, fake, fake, fake, fake, fake)
    assert L.tp_conv_backward_fc(cg.handle, ctypes.byref(g), *args, 2, fake, 1 << 30, None) == -1
    assert "flags" in L.tp_conv_last_error().decode()
    assert L.tp_conv_backward_fc(cg.handle, ctypes.byref(g), *args, tpc.TP_FC_STATE_SAVED, fake,
                                 need - 1, None) == -5
    assert L.tp_conv_backward_fc(cg.handle, ctypes.byref(g), *args, 0, odd, 1 << 30, None) == -1
    assert L.tp_conv_backward_fc(cg.handle, ctypes.byref(gg), *args, 0, fake, 1 << 30, None) == -1
    assert L.tp_conv_backward_fc(p.handle, ctypes.byref(g), *args, 0, fake, 1 << 30, None) == -3


def test_second_order_and_edge_vector_argument_errors_without_launch():
    """Host validation of the radial and fully connected second-order backward
    and of the edge-vector entry points: each case returns its status before
    any HIP call."""
    L = tpc.lib()
    fake = ctypes.c_void_p(0x1000)
    odd = ctypes.c_void_p(0x1004)                  # not 16-byte aligned
    plain = tpc.Plan("16x0e+16x1o+16x2e", 2, 2)
    rad = tpc.Plan("16x0e+16x1o+16x2e", 2, 2, radial=(8, 64, 5.0), uvw=True)
    g = tpc._Graph(4, 10, fake, fake, fake, fake, fake, fake)
    sz = ctypes.c_size_t()
    # radial second order: workspace, then the entry point
    assert L.tp_conv_radial_double_workspace(plain.handle, 4, 0, ctypes.byref(sz)) == -3
    assert L.tp_conv_radial_double_workspace(rad.handle, -1, 0, ctypes.byref(sz)) == -1
    assert L.tp_conv_radial_double_workspace(rad.handle, 4, 0, ctypes.byref(sz)) == 0 and sz.value > 0
    base = sz.value
    assert L.tp_conv_radial_double_workspace(rad.handle, 4, 1, ctypes.byref(sz)) == 0 and sz.value > base
    # x, Y, r_len, W1, W2 | Wmix | grad_out | gg_x, gg_Y, gg_rlen | d_x, d_Y, d_rlen, d_W1, d_W2 | d_Wmix | d_g
    args = [fake] * 5 + [None] + [fake] + [fake] * 3 + [fake] * 5 + [None] + [fake]
    f = L.tp_conv_double_backward_radial
    assert f(None, ctypes.byref(g), *args, fake, 1 << 30, None) == -1
    assert f(plain.handle, ctypes.byref(g), *args, fake, 1 << 30, None) == -3
    assert f(rad.handle, ctypes.byref(g), *args, fake, 16, None) == -5
    bad = list(args)
    bad[7] = odd                                   # gg_x
    assert f(rad.handle, ctypes.byref(g), *bad, fake, 1 << 30, None) == -1
    assert "aligned" in L.tp_conv_last_error().decode()
    nomix = list(args)
    nomix[15] = fake                               # d_Wmix without Wmix
    assert f(rad.handle, ctypes.byref(g), *nomix, fake, 1 << 30, None) == -1
    noy = list(args)
    noy[1] = None                                  # Y with edges
    assert f(rad.handle, ctypes.byref(g), *noy, fake, 1 << 30, None) == -1
    # fully connected second order
    assert L.tp_conv_fc_double_workspace(plain.handle, 4, 10, 3, ctypes.byref(sz)) == -3
    assert L.tp_conv_fc_double_workspace(plain.handle, -1, 10, 8, ctypes.byref(sz)) == -1
    assert L.tp_conv_fc_double_workspace(plain.handle, 4, 10, 8, ctypes.byref(sz)) == 0 and sz.value > 0
    # x, Y, R | H | Theta, grad_out | gg_x, gg_Y, gg_R, gg_Theta | d_x, d_Y, d_R, d_Theta, d_g
    fd = L.tp_conv_double_backward_fc
    fargs = [fake] * 3 + [8] + [fake] * 2 + [fake] * 4 + [fake] * 5
    assert fd(plain.handle, ctypes.byref(g), *fargs, fake, 16, None) == -5
    bad = list(fargs)
    bad[9] = odd                                   # gg_Theta
    assert fd(plain.handle, ctypes.byref(g), *bad, fake, 1 << 30, None) == -1
    bad = list(fargs)
    bad[5] = None                                  # grad_out
    assert fd(plain.handle, ctypes.byref(g), *bad, fake, 1 << 30, None) == -1
    bad = list(fargs)
    bad[3] = 3                                     # radial features not compiled
    assert fd(plain.handle, ctypes.byref(g), *bad, fake, 1 << 30, None) == -3
    # edge-vector forms
    assert L.tp_conv_forward_r(plain.handle, ctypes.byref(g), odd, fake, fake, fake, None) == -1
    assert L.tp_conv_forward_r(plain.handle, ctypes.byref(g), fake, None, fake, fake, None) == -1
    assert L.tp_conv_backward_r(plain.handle, ctypes.byref(g), fake, fake, fake, odd, fake, fake, fake,
                                None) == -1
    assert L.tp_conv_forward_radial_r(plain.handle, ctypes.byref(g), fake, fake, fake, fake, None, None,
                                      fake, None) == -3


def test_gaunt_second_order_argument_errors_without_launch():
    L = tpc.lib()
    fake = ctypes.c_void_p(0x1000)
    odd = ctypes.c_void_p(0x1004)
    plain = tpc.Plan("16x0e+16x1o+16x2e", 2, 2)
    gaunt = tpc.Plan("16x0e+16x1o+16x2e", 2, 2, mode=tpc.TP_MODE_GAUNT)
    g = tpc._Graph(4, 10, fake, fake, fake, fake, fake, fake)
    sz = ctypes.c_size_t()
    assert L.tp_conv_gaunt_double_workspace(plain.handle, 4, 10, ctypes.byref(sz)) == -3
    assert L.tp_conv_gaunt_double_workspace(gaunt.handle, 4, -1, ctypes.byref(sz)) == -1
    assert L.tp_conv_gaunt_double_workspace(gaunt.handle, 4, 10, ctypes.byref(sz)) == 0
    # d_grad_out, d_x, d_Y, d_w rows: 4 x 144, 4 x 144, 10 x 9, 10 x 48 floats, each 256-byte aligned
    assert sz.value == 4 * (576 + 576 + 128 + 512)
    # x, Y, w, grad_out | gg_x, gg_Y, gg_w | d_x, d_Y, d_w, d_g
    args = [fake] * 4 + [fake] * 3 + [fake] * 4
    f = L.tp_conv_double_backward_gaunt
    assert f(None, ctypes.byref(g), *args, fake, 1 << 30, None) == -1
    assert f(plain.handle, ctypes.byref(g), *args, fake, 1 << 30, None) == -3
    assert f(gaunt.handle, ctypes.byref(g), *args, fake, 16, None) == -5
    bad = list(args)
    bad[6] = odd                                   # gg_w
    assert f(gaunt.handle, ctypes.byref(g), *bad, fake, 1 << 30, None) == -1
    bad = list(args)
    bad[3] = None                                  # grad_out
    assert f(gaunt.handle, ctypes.byref(g), *bad, fake, 1 << 30, None) == -1


def test_radial_lmax3_plans_without_launch():
    """The lmax-3 radial layer is compiled for 16, 32 and 64 channels; other
    widths are refused at plan time; its workspace queries (first and second
    order) answer, and the second-order entry point validates like the lmax-2
    one (before any HIP call)."""
    L = tpc.lib()
    fake = ctypes.c_void_p(0x1000)
    for U in (16, 32, 64):
        p = tpc.Plan(f"{U}x0e+{U}x1o+{U}x2e+{U}x3o", 3, 3, radial=(8, 64, 5.0), uvw=True)
        sz = ctypes.c_size_t()
        assert L.tp_conv_radial_workspace(p.handle, 100, 1, ctypes.byref(sz)) == 0 and sz.value > 0
        assert L.tp_conv_radial_double_workspace(p.handle, 100, 0, ctypes.byref(sz)) == 0 and sz.value > 0
        g = tpc._Graph(4, 10, fake, fake, fake, fake, fake, fake)
        args = [fake] * 5 + [None] + [fake] + [fake] * 3 + [fake] * 5 + [None] + [fake]
        assert L.tp_conv_double_backward_radial(p.handle, ctypes.byref(g), *args, fake, 16, None) == -5
    with pytest.raises(Exception, match="radial"):
        tpc.Plan("128x0e+128x1o+128x2e+128x3o", 3, 3, radial=(8, 64, 5.0))
    with pytest.raises(Exception, match="radial"):
        tpc.Plan("16x0e+16x1o+16x2e+16x3o", 3, 3, radial=(8, 32, 5.0))


def test_sender_layout_argument_errors_without_launch():
    """The sender-grouped layout's entry points reject bad arguments on the
    host: missing e_pos or sender grouping, misaligned rows, and a signature
    without a one-pass backward (0e+1o+2e+3o / lmax 3)."""
    L = tpc.lib()
    p = tpc.Plan("8x0e+8x1o", 2, 2)
    p3 = tpc.Plan("16x0e+16x1o+16x2e+16x3o", 3, 3)
    fake, odd = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x1004)
    g = tpc._Graph(4, 10, fake, fake, fake, fake, fake, fake)
    no_sender = tpc._Graph(4, 10, fake, fake, fake, None, None, None)
    assert L.tp_conv_graph_sender_positions(ctypes.byref(g), None, None) == -1
    assert L.tp_conv_graph_sender_positions(ctypes.byref(no_sender), fake, None) == -1
    assert L.tp_conv_graph_sender_positions(None, fake, None) == -1
    # forward: e_pos is required when there are edges
    assert L.tp_conv_forward_sg(p.handle, ctypes.byref(g), None, fake, fake, fake, fake, None) == -1
    assert "e_pos" in L.tp_conv_last_error().decode()
    assert L.tp_conv_forward_sg(p.handle, ctypes.byref(g), fake, odd, fake, fake, fake, None) == -1
    assert "16-byte" in L.tp_conv_last_error().decode()
    assert L.tp_conv_forward_sg(None, ctypes.byref(g), fake, fake, fake, fake, fake, None) == -1
    # backward: needs the sender grouping and aligned x, w, grad_out
    assert L.tp_conv_backward_sg(p.handle, ctypes.byref(no_sender), fake, fake, fake, fake, fake, fake,
                                 fake, None) == -1
    for bad in (0, 2, 3):
        args = [fake] * 4
        args[bad] = odd
        assert L.tp_conv_backward_sg(p.handle, ctypes.byref(g), *args, fake, fake, fake, None) == -1
        assert "16-byte" in L.tp_conv_last_error().decode()
    assert L.tp_conv_backward_sg(p3.handle, ctypes.byref(g), fake, fake, fake, fake, fake, fake, fake,
                                 None) == -3
    assert "one-pass" in L.tp_conv_last_error().decode()
    # nothing requested: returns before any launch
    assert L.tp_conv_backward_sg(p.handle, ctypes.byref(g), fake, fake, fake, fake, None, None, None,
                                 None) == 0


def test_launch_order_argument_errors_without_launch():
    """tp_conv_graph_launch_order checks its graph, outputs and workspace on the
    host; the graph struct carries the optional order fields at its end."""
    L = tpc.lib()
    assert [f[0] for f in tpc._Graph._fields_][-2:] == ["order", "t_order"]
    fake = ctypes.c_void_p(0x1000)
    need = ctypes.c_size_t()
    assert L.tp_conv_graph_order_workspace(1000, ctypes.byref(need)) == 0 and need.value >= 4000
    assert L.tp_conv_graph_order_workspace(-1, ctypes.byref(need)) == -1
    g = tpc._Graph(4, 10, fake, fake, fake, fake, fake, fake)
    no_sender = tpc._Graph(4, 10, fake, fake, fake, None, None, None)
    assert L.tp_conv_graph_launch_order(ctypes.byref(g), None, None, fake, 1 << 20, None) == -1
    assert L.tp_conv_graph_launch_order(ctypes.byref(g), fake, fake, fake, 16, None) == -5
    assert L.tp_conv_graph_launch_order(ctypes.byref(g), fake, fake, None, 1 << 20, None) == -5
    assert L.tp_conv_graph_launch_order(ctypes.byref(no_sender), fake, fake, fake, 1 << 20, None) == -1
    assert L.tp_conv_graph_launch_order(None, fake, fake, fake, 1 << 20, None) == -1
