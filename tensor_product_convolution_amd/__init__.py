"""Python binding of libtpconv (MI355X / gfx950 tensor-product convolution).

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream; results are torch
tensors on the same device.  There is no fallback: if ``libtpconv.so`` is
missing or no GPU is present the calls raise.

Conventions, layouts and error codes are those of ``include/tpconv.h``.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libtpconv.so")

TP_OK = 0
STATUS_NAMES = {-1: "TP_ERR_ARG", -2: "TP_ERR_IRREPS", -3: "TP_ERR_UNSUPPORTED",
                -4: "TP_ERR_OVERFLOW", -5: "TP_ERR_WORKSPACE", -6: "TP_ERR_HIP",
                -7: "TP_ERR_INDEX"}
TP_GRAPH_CHECK = 1
TP_MODE_UVU, TP_MODE_GAUNT = 0, 1
TP_FC_STATE_SAVED = 1

# every exported symbol of include/tpconv.h
EXPORTS = (
    "tp_conv_plan_create", "tp_conv_plan_info", "tp_conv_plan_paths", "tp_conv_plan_cg",
    "tp_conv_plan_destroy", "tp_cg_real", "tp_conv_graph_workspace", "tp_conv_graph_build",
    "tp_conv_graph_build_static", "tp_conv_gather_rows", "tp_conv_sph_harm", "tp_conv_forward", "tp_conv_backward",
    "tp_conv_forward_r", "tp_conv_backward_r",
    "tp_conv_graph_sender_positions", "tp_conv_forward_sg", "tp_conv_backward_sg",
    "tp_conv_graph_order_workspace", "tp_conv_graph_launch_order",
    "tp_conv_uvw_forward", "tp_conv_uvw_backward", "tp_conv_uvw_workspace",
    "tp_conv_forward_radial", "tp_conv_backward_radial", "tp_conv_radial_workspace",
    "tp_conv_forward_radial_r", "tp_conv_backward_radial_r", "tp_conv_double_backward_radial",
    "tp_conv_radial_double_workspace", "tp_conv_sph_harm_backward", "tp_conv_double_backward", "tp_conv_fc_workspace",
    "tp_conv_forward_fc", "tp_conv_fc_backward_workspace", "tp_conv_backward_fc", "tp_conv_fc_double_workspace",
    "tp_conv_double_backward_fc", "tp_conv_gaunt_dims", "tp_conv_forward_gaunt", "tp_conv_backward_gaunt",
    "tp_conv_gaunt_double_workspace", "tp_conv_double_backward_gaunt",
    "tp_conv_last_error",
)


class TPError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class _Graph(ctypes.Structure):
    _fields_ = [("n_nodes", ctypes.c_int32), ("n_edges", ctypes.c_int32),
                ("row_ptr", ctypes.c_void_p), ("col", ctypes.c_void_p),
                ("perm", ctypes.c_void_p), ("t_row_ptr", ctypes.c_void_p),
                ("t_perm", ctypes.c_void_p), ("t_col", ctypes.c_void_p),
                ("order", ctypes.c_void_p), ("t_order", ctypes.c_void_p)]


class _Opts(ctypes.Structure):
    _fields_ = [("radial_basis", ctypes.c_int32), ("radial_hidden", ctypes.c_int32),
                ("r_cut", ctypes.c_float), ("uvw", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded ctypes library (loads on first use; raises if not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                           "python tensor_product_convolution_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, VP = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                           ctypes.c_size_t, ctypes.c_void_p)
    pI32 = ctypes.POINTER(ctypes.c_int32)
    sig = {
        "tp_conv_plan_create": (I32, [ctypes.POINTER(P), ctypes.c_char_p, I32, I32, I32,
                                      ctypes.POINTER(_Opts)]),
        "tp_conv_plan_info": (I32, [P, pI32, pI32, pI32, pI32, pI32, pI32, ctypes.c_char_p, SZ]),
        "tp_conv_plan_paths": (I32, [P, VP]),
        "tp_conv_plan_cg": (I32, [P, VP, VP]),
        "tp_conv_plan_destroy": (None, [P]),
        "tp_cg_real": (I32, [I32, I32, I32, VP]),
        "tp_conv_graph_workspace": (I32, [I32, I32, ctypes.POINTER(SZ)]),
        "tp_conv_graph_build": (I32, [VP, VP, I32, I32, VP, VP, VP, VP, VP, VP, VP, SZ, I32, VP]),
        "tp_conv_graph_build_static": (I32, [VP, VP, I32, I32, VP, VP, VP, VP, VP, VP, I32, VP]),
        "tp_conv_gather_rows": (I32, [VP, VP, I64, I64, VP, VP]),
        "tp_conv_sph_harm": (I32, [I32, VP, I32, VP, VP]),
        "tp_conv_forward": (I32, [P, ctypes.POINTER(_Graph), VP, VP, VP, VP, VP]),
        "tp_conv_backward": (I32, [P, ctypes.POINTER(_Graph), VP, VP, VP, VP, VP, VP, VP, VP]),
        "tp_conv_forward_r": (I32, [P, ctypes.POINTER(_Graph), VP, VP, VP, VP, VP]),
        "tp_conv_backward_r": (I32, [P, ctypes.POINTER(_Graph), VP, VP, VP, VP, VP, VP, VP, VP]),
        "tp_conv_graph_sender_positions": (I32, [ctypes.POINTER(_Graph), VP, VP]),
        "tp_conv_graph_order_workspace": (I32, [I32, ctypes.POINTER(SZ)]),
        "tp_conv_graph_launch_order": (I32, [ctypes.POINTER(_Graph), VP, VP, VP, SZ, VP]),
        "tp_conv_forward_sg": (I32, [P, ctypes.POINTER(_Graph), VP, VP, VP, VP, VP, VP]),
        "tp_conv_backward_sg": (I32, [P, ctypes.POINTER(_Graph), VP, VP, VP, VP, VP, VP, VP, VP]),
        "tp_conv_uvw_forward": (I32, [P, I32, VP, VP, VP, VP]),
        "tp_conv_uvw_backward": (I32, [P, I32, VP, VP, VP, VP, VP, VP, SZ, VP]),
        "tp_conv_uvw_workspace": (I32, [P, ctypes.POINTER(SZ)]),
        "tp_conv_forward_radial": (I32, [P, ctypes.POINTER(_Graph), VP, VP, VP, VP, VP, VP, VP, VP,
                                         VP]),
        "tp_conv_backward_radial": (I32, [P, ctypes.POINTER(_Graph), VP, VP, VP, VP, VP, VP, VP,
                                          VP, VP, VP, VP, VP, VP, VP, VP, SZ, VP]),
        "tp_conv_sph_harm_backward": (I32, [I32, VP, I32, VP, VP, VP, VP]),
        "tp_conv_forward_radial_r": (I32, [P, ctypes.POINTER(_Graph), VP, VP, VP, VP, VP, VP, VP, VP]),
        "tp_conv_backward_radial_r": (I32, [P, ctypes.POINTER(_Graph), VP, VP, VP, VP, VP, VP, VP, VP,
                                            VP, VP, VP, VP, VP, SZ, VP]),
        "tp_conv_fc_workspace": (I32, [P, I32, I32, ctypes.POINTER(SZ)]),
        "tp_conv_forward_fc": (I32, [P, ctypes.POINTER(_Graph), VP, VP, VP, I32, VP, VP, VP, SZ, VP]),
        "tp_conv_fc_backward_workspace": (I32, [P, I32, I32, ctypes.POINTER(SZ)]),
        "tp_conv_backward_fc": (I32, [P, ctypes.POINTER(_Graph), VP, VP, VP, I32, VP, VP, VP, VP, VP, VP, I32,
                                      VP, SZ, VP]),
        "tp_conv_fc_double_workspace": (I32, [P, I32, I32, I32, ctypes.POINTER(SZ)]),
        "tp_conv_double_backward_fc": (I32, [P, ctypes.POINTER(_Graph), VP, VP, VP, I32] + [VP] * 11
                                       + [VP, SZ, VP]),
        "tp_conv_gaunt_double_workspace": (I32, [P, I32, I32, ctypes.POINTER(SZ)]),
        "tp_conv_double_backward_gaunt": (I32, [P, ctypes.POINTER(_Graph)] + [VP] * 11 + [VP, SZ, VP]),
        "tp_conv_gaunt_dims": (I32, [P, ctypes.POINTER(I32), ctypes.POINTER(I32), ctypes.POINTER(I32)]),
        "tp_conv_forward_gaunt": (I32, [P, ctypes.POINTER(_Graph), VP, VP, VP, VP, VP]),
        "tp_conv_backward_gaunt": (I32, [P, ctypes.POINTER(_Graph), VP, VP, VP, VP, VP, VP, VP, VP]),
        "tp_conv_double_backward": (I32, [P, ctypes.POINTER(_Graph), VP, VP, VP, VP, VP, VP, VP, VP,
                                          VP, VP, VP, VP]),
        "tp_conv_radial_workspace": (I32, [P, I32, I32, ctypes.POINTER(SZ)]),
        "tp_conv_double_backward_radial": (I32, [P, ctypes.POINTER(_Graph)] + [VP] * 18 + [SZ, VP]),
        "tp_conv_radial_double_workspace": (I32, [P, I32, I32, ctypes.POINTER(SZ)]),
        "tp_conv_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _check(status):
    if status != TP_OK:
        raise TPError(status, lib().tp_conv_last_error().decode())


def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def cg_real(l1, l2, l3):
    """Dense real CG tensor [2l1+1, 2l2+1, 2l3+1] from the library's builder (host)."""
    out = np.zeros((2 * l1 + 1) * (2 * l2 + 1) * (2 * l3 + 1), dtype=np.float64)
    _check(lib().tp_cg_real(l1, l2, l3, out.ctypes.data_as(ctypes.c_void_p)))
    return out.reshape(2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1)


class Plan:
    """Paths, output irreps and CG tables of a channel-wise product (host only)."""

    def __init__(self, irreps_in, lmax_sh, lmax_out, mode=0, radial=None, uvw=False):
        """radial: (n_basis, hidden, r_cut) for radial-network edge weights."""
        h = ctypes.c_void_p()
        opts = None
        if radial is not None or uvw:
            nb, nh, rc = radial if radial is not None else (0, 0, 0.0)
            opts = ctypes.byref(_Opts(nb, nh, rc, 1 if uvw else 0))
        _check(lib().tp_conv_plan_create(ctypes.byref(h), irreps_in.encode(), lmax_sh, lmax_out,
                                         mode, opts))
        self.radial = radial
        self.uvw = uvw
        self._h = h
        self.irreps_in = irreps_in
        self.lmax_sh, self.lmax_out = lmax_sh, lmax_out
        v = [ctypes.c_int32() for _ in range(6)]
        buf = ctypes.create_string_buffer(256)
        _check(lib().tp_conv_plan_info(h, *[ctypes.byref(x) for x in v], buf, 256))
        (self.n_paths, self.mul, self.xdim, self.ysh, self.outdim, self.nnz) = [x.value for x in v]
        self.out_irreps = buf.value.decode()

    @property
    def handle(self):
        return self._h

    def paths(self):
        a = np.zeros(4 * self.n_paths, dtype=np.int32)
        _check(lib().tp_conv_plan_paths(self._h, a.ctypes.data_as(ctypes.c_void_p)))
        return [tuple(int(v) for v in r) for r in a.reshape(-1, 4)]

    def cg(self):
        idx = np.zeros(4 * self.nnz, dtype=np.int16)
        val = np.zeros(self.nnz, dtype=np.float64)
        _check(lib().tp_conv_plan_cg(self._h, idx.ctypes.data_as(ctypes.c_void_p),
                                     val.ctypes.data_as(ctypes.c_void_p)))
        return idx.reshape(-1, 4), val

    def dims(self):
        return dict(xdim=self.xdim, n_paths=self.n_paths, U=self.mul, outdim=self.outdim,
                    n_out_irreps=len(self.out_irreps.split("+")))

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().tp_conv_plan_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Graph:
    """Receiver/sender grouping of an edge list (int32 device tensors)."""

    def __init__(self, n_nodes, n_edges, row_ptr, col, perm, t_row_ptr, t_perm, t_col):
        self.n_nodes, self.n_edges = n_nodes, n_edges
        self.row_ptr, self.col, self.perm = row_ptr, col, perm
        self.t_row_ptr, self.t_perm, self.t_col = t_row_ptr, t_perm, t_col
        self.order = self.t_order = None        # launch orders (graph_launch_order)

    def cstruct(self):
        ptr = lambda t: None if t is None else t.data_ptr()
        return _Graph(self.n_nodes, self.n_edges, self.row_ptr.data_ptr(),
                      self.col.data_ptr(), self.perm.data_ptr(), self.t_row_ptr.data_ptr(),
                      self.t_perm.data_ptr(), self.t_col.data_ptr(), ptr(self.order),
                      ptr(self.t_order))


def graph_build(src, dst, n_nodes, check=True):
    """Group edges src -> dst (int32 cuda tensors) by receiver and by sender."""
    torch = _torch()
    _need(src, "src", torch.int32)
    E = src.shape[0]
    _need(dst, "dst", torch.int32, (E,))
    dev = src.device
    need = ctypes.c_size_t()
    _check(lib().tp_conv_graph_workspace(n_nodes, E, ctypes.byref(need)))
    ws = torch.empty(need.value, dtype=torch.uint8, device=dev)
    i32 = dict(dtype=torch.int32, device=dev)
    g = Graph(n_nodes, E, torch.empty(n_nodes + 1, **i32), torch.empty(E, **i32),
              torch.empty(E, **i32), torch.empty(n_nodes + 1, **i32),
              torch.empty(E, **i32), torch.empty(E, **i32))
    _check(lib().tp_conv_graph_build(_ptr(src), _ptr(dst), E, n_nodes, _ptr(g.row_ptr),
                                     _ptr(g.col), _ptr(g.perm), _ptr(g.t_row_ptr),
                                     _ptr(g.t_perm), _ptr(g.t_col), _ptr(ws), need.value,
                                     TP_GRAPH_CHECK if check else 0, _stream(dev)))
    g._ws = ws
    return g


def graph_build_static(src, dst, n_nodes, check=True, out=None):
    """graph_build through the entry point that allocates nothing (the
    library's static scratch); ``out`` (a Graph of the right sizes) is
    filled in place, else new arrays are made."""
    torch = _torch()
    _need(src, "src", torch.int32)
    E = src.shape[0]
    _need(dst, "dst", torch.int32, (E,))
    dev = src.device
    i32 = dict(dtype=torch.int32, device=dev)
    g = out or Graph(n_nodes, E, torch.empty(n_nodes + 1, **i32), torch.empty(E, **i32),
                     torch.empty(E, **i32), torch.empty(n_nodes + 1, **i32),
                     torch.empty(E, **i32), torch.empty(E, **i32))
    _check(lib().tp_conv_graph_build_static(_ptr(src), _ptr(dst), E, n_nodes, _ptr(g.row_ptr),
                                            _ptr(g.col), _ptr(g.perm), _ptr(g.t_row_ptr),
                                            _ptr(g.t_perm), _ptr(g.t_col),
                                            TP_GRAPH_CHECK if check else 0, _stream(dev)))
    return g


def gather_rows(t, perm, out=None):
    """out[q] = t[perm[q]] for a contiguous 4-byte-element tensor t (rows = dim 0)."""
    torch = _torch()
    _need(perm, "perm", torch.int32)
    if t.element_size() != 4 or not t.is_contiguous():
        raise TypeError("gather_rows needs a contiguous tensor of 4-byte elements")
    n = perm.shape[0]
    words = int(t[0].numel()) if t.shape[0] else 0
    if out is None:
        out = torch.empty((n,) + tuple(t.shape[1:]), dtype=t.dtype, device=t.device)
    _check(lib().tp_conv_gather_rows(_ptr(t), _ptr(perm), n, words, _ptr(out), _stream(t.device)))
    return out


def sph_harm(lmax, r, out=None):
    """Real component-normalised harmonics of the rows of r [E, 3] (float32 cuda)."""
    torch = _torch()
    _need(r, "r", torch.float32)
    E = r.shape[0]
    if out is None:
        out = torch.empty((E, (lmax + 1) ** 2), dtype=torch.float32, device=r.device)
    _check(lib().tp_conv_sph_harm(lmax, _ptr(r), E, _ptr(out), _stream(r.device)))
    return out


def sph_harm_backward(lmax, r, grad_Y, grad_rlen=None, out=None):
    """grad_r [E, 3] = grad_Y . dY/dr (+ grad_rlen * r/|r|) for Y = sph_harm(lmax, r)."""
    torch = _torch()
    _need(r, "r", torch.float32)
    E = r.shape[0]
    _need(grad_Y, "grad_Y", torch.float32, (E, (lmax + 1) ** 2))
    if grad_rlen is not None:
        _need(grad_rlen, "grad_rlen", torch.float32, (E,))
    if out is None:
        out = torch.empty((E, 3), dtype=torch.float32, device=r.device)
    _check(lib().tp_conv_sph_harm_backward(lmax, _ptr(r), E, _ptr(grad_Y), _ptr(grad_rlen), _ptr(out),
                                           _stream(r.device)))
    return out


def forward(plan, graph, x, Y, w, out=None):
    """out [N, outdim] of the convolution (edge arrays in receiver-sorted order)."""
    torch = _torch()
    N, E = graph.n_nodes, graph.n_edges
    _need(x, "x", torch.float32, (N, plan.xdim))
    _need(Y, "Y", torch.float32, (E, plan.ysh))
    _need(w, "w", torch.float32, (E, plan.n_paths, plan.mul))
    if out is None:
        out = torch.empty((N, plan.outdim), dtype=torch.float32, device=x.device)
    _need(out, "out", torch.float32, (N, plan.outdim))
    g = graph.cstruct()
    _check(lib().tp_conv_forward(plan.handle, ctypes.byref(g), _ptr(x), _ptr(Y), _ptr(w),
                                 _ptr(out), _stream(x.device)))
    return out


def backward(plan, graph, x, Y, w, grad_out, want=("x", "Y", "w"), outs=None):
    """(grad_x, grad_Y, grad_w); entries not in ``want`` come back as None."""
    torch = _torch()
    N, E = graph.n_nodes, graph.n_edges
    _need(x, "x", torch.float32, (N, plan.xdim))
    _need(Y, "Y", torch.float32, (E, plan.ysh))
    _need(w, "w", torch.float32, (E, plan.n_paths, plan.mul))
    _need(grad_out, "grad_out", torch.float32, (N, plan.outdim))
    f32 = dict(dtype=torch.float32, device=x.device)
    if outs is None:
        gx = torch.empty((N, plan.xdim), **f32) if "x" in want else None
        gY = torch.empty((E, plan.ysh), **f32) if "Y" in want else None
        gw = torch.empty((E, plan.n_paths, plan.mul), **f32) if "w" in want else None
    else:
        gx, gY, gw = outs
    g = graph.cstruct()
    _check(lib().tp_conv_backward(plan.handle, ctypes.byref(g), _ptr(x), _ptr(Y), _ptr(w),
                                  _ptr(grad_out), _ptr(gx), _ptr(gY), _ptr(gw),
                                  _stream(x.device)))
    return gx, gY, gw


def graph_launch_order(graph, receivers=True, senders=True):
    """Fill graph.order / graph.t_order (int32 [N]): nodes by descending in- /
    out-degree, ties by node id; the convolution calls on this graph then
    launch their workgroups in that order (results unchanged)."""
    torch = _torch()
    N = graph.n_nodes
    dev = graph.row_ptr.device
    need = ctypes.c_size_t()
    _check(lib().tp_conv_graph_order_workspace(N, ctypes.byref(need)))
    ws = torch.empty(max(need.value, 1), dtype=torch.uint8, device=dev)
    order = torch.empty(N, dtype=torch.int32, device=dev) if receivers else None
    t_order = torch.empty(N, dtype=torch.int32, device=dev) if senders else None
    g = graph.cstruct()
    _check(lib().tp_conv_graph_launch_order(ctypes.byref(g), _ptr(order), _ptr(t_order), _ptr(ws),
                                            need.value, _stream(dev)))
    graph.order, graph.t_order = order, t_order
    return graph


def graph_sender_positions(graph, out=None):
    """e_pos [E] int32: the sender-grouped position of each receiver-sorted edge."""
    torch = _torch()
    E = graph.n_edges
    dev = graph.row_ptr.device
    if out is None:
        out = torch.empty(E, dtype=torch.int32, device=dev)
    _need(out, "e_pos", torch.int32, (E,))
    g = graph.cstruct()
    _check(lib().tp_conv_graph_sender_positions(ctypes.byref(g), _ptr(out), _stream(dev)))
    return out


def forward_sg(plan, graph, e_pos, x, Y, w, out=None):
    """forward with Y and w in the sender grouping (row k = sender-grouped position k)."""
    torch = _torch()
    N, E = graph.n_nodes, graph.n_edges
    _need(e_pos, "e_pos", torch.int32, (E,))
    _need(x, "x", torch.float32, (N, plan.xdim))
    _need(Y, "Y", torch.float32, (E, plan.ysh))
    _need(w, "w", torch.float32, (E, plan.n_paths, plan.mul))
    if out is None:
        out = torch.empty((N, plan.outdim), dtype=torch.float32, device=x.device)
    _need(out, "out", torch.float32, (N, plan.outdim))
    g = graph.cstruct()
    _check(lib().tp_conv_forward_sg(plan.handle, ctypes.byref(g), _ptr(e_pos), _ptr(x), _ptr(Y),
                                    _ptr(w), _ptr(out), _stream(x.device)))
    return out


def backward_sg(plan, graph, x, Y, w, grad_out, want=("x", "Y", "w"), outs=None):
    """(grad_x, grad_Y, grad_w) with every edge array in the sender grouping."""
    torch = _torch()
    N, E = graph.n_nodes, graph.n_edges
    _need(x, "x", torch.float32, (N, plan.xdim))
    _need(Y, "Y", torch.float32, (E, plan.ysh))
    _need(w, "w", torch.float32, (E, plan.n_paths, plan.mul))
    _need(grad_out, "grad_out", torch.float32, (N, plan.outdim))
    f32 = dict(dtype=torch.float32, device=x.device)
    if outs is None:
        gx = torch.empty((N, plan.xdim), **f32) if "x" in want else None
        gY = torch.empty((E, plan.ysh), **f32) if "Y" in want else None
        gw = torch.empty((E, plan.n_paths, plan.mul), **f32) if "w" in want else None
    else:
        gx, gY, gw = outs
    g = graph.cstruct()
    _check(lib().tp_conv_backward_sg(plan.handle, ctypes.byref(g), _ptr(x), _ptr(Y), _ptr(w),
                                     _ptr(grad_out), _ptr(gx), _ptr(gY), _ptr(gw),
                                     _stream(x.device)))
    return gx, gY, gw


def forward_r(plan, graph, x, r, w, out=None):
    """forward from the edge vectors r [E, 3] (receiver-sorted); harmonics on chip."""
    torch = _torch()
    N, E = graph.n_nodes, graph.n_edges
    _need(x, "x", torch.float32, (N, plan.xdim))
    _need(r, "r", torch.float32, (E, 3))
    _need(w, "w", torch.float32, (E, plan.n_paths, plan.mul))
    if out is None:
        out = torch.empty((N, plan.outdim), dtype=torch.float32, device=x.device)
    _need(out, "out", torch.float32, (N, plan.outdim))
    g = graph.cstruct()
    _check(lib().tp_conv_forward_r(plan.handle, ctypes.byref(g), _ptr(x), _ptr(r), _ptr(w),
                                   _ptr(out), _stream(x.device)))
    return out


def backward_r(plan, graph, x, r, w, grad_out, want=("x", "r", "w"), outs=None):
    """(grad_x, grad_r, grad_w) of forward_r; entries not in ``want`` come back as None."""
    torch = _torch()
    N, E = graph.n_nodes, graph.n_edges
    _need(x, "x", torch.float32, (N, plan.xdim))
    _need(r, "r", torch.float32, (E, 3))
    _need(w, "w", torch.float32, (E, plan.n_paths, plan.mul))
    _need(grad_out, "grad_out", torch.float32, (N, plan.outdim))
    f32 = dict(dtype=torch.float32, device=x.device)
    if outs is None:
        gx = torch.empty((N, plan.xdim), **f32) if "x" in want else None
        gr = torch.empty((E, 3), **f32) if "r" in want else None
        gw = torch.empty((E, plan.n_paths, plan.mul), **f32) if "w" in want else None
    else:
        gx, gr, gw = outs
    g = graph.cstruct()
    _check(lib().tp_conv_backward_r(plan.handle, ctypes.byref(g), _ptr(x), _ptr(r), _ptr(w),
                                    _ptr(grad_out), _ptr(gx), _ptr(gr), _ptr(gw), _stream(x.device)))
    return gx, gr, gw


def double_backward(plan, graph, x, Y, w, grad_out, gg_x=None, gg_Y=None, gg_w=None,
                    want=("x", "Y", "w", "g")):
    """(d_x, d_Y, d_w, d_grad_out): gradients of <gg_x, grad_x> + <gg_Y, grad_Y> +
    <gg_w, grad_w> with respect to the inputs of backward(); missing cotangents are
    zero, outputs not in ``want`` are None."""
    torch = _torch()
    N, E = graph.n_nodes, graph.n_edges
    _need(x, "x", torch.float32, (N, plan.xdim))
    _need(Y, "Y", torch.float32, (E, plan.ysh))
    _need(w, "w", torch.float32, (E, plan.n_paths, plan.mul))
    _need(grad_out, "grad_out", torch.float32, (N, plan.outdim))
    for t, n, like in ((gg_x, "gg_x", x), (gg_Y, "gg_Y", Y), (gg_w, "gg_w", w)):
        if t is not None:
            _need(t, n, torch.float32, tuple(like.shape))
    dx = torch.empty_like(x) if "x" in want else None
    dY = torch.empty_like(Y) if "Y" in want else None
    dw = torch.empty_like(w) if "w" in want else None
    dg = torch.empty_like(grad_out) if "g" in want else None
    gs = graph.cstruct()
    _check(lib().tp_conv_double_backward(plan.handle, ctypes.byref(gs), _ptr(x), _ptr(Y), _ptr(w),
                                         _ptr(grad_out), _ptr(gg_x), _ptr(gg_Y), _ptr(gg_w),
                                         _ptr(dx), _ptr(dY), _ptr(dw), _ptr(dg), _stream(x.device)))
    return dx, dY, dw, dg


def fc_workspace(plan, n_nodes, n_radial):
    """bytes of the node-sized receiver state forward_fc needs"""
    b = ctypes.c_size_t()
    _check(lib().tp_conv_fc_workspace(plan.handle, n_nodes, n_radial, ctypes.byref(b)))
    return b.value


def forward_fc(plan, graph, x, Y, R, Theta, out=None, ws=None):
    """out [N, outdim] of the convolution with fully connected per-edge weights
    W_e = sum_h R[e, h] Theta[h] (R receiver-sorted [E, H], Theta [H, P, U, U])."""
    torch = _torch()
    N, E = graph.n_nodes, graph.n_edges
    H = R.shape[1]
    _need(x, "x", torch.float32, (N, plan.xdim))
    _need(Y, "Y", torch.float32, (E, plan.ysh))
    _need(R, "R", torch.float32, (E, H))
    _need(Theta, "Theta", torch.float32, (H, plan.n_paths, plan.mul, plan.mul))
    if out is None:
        out = torch.empty((N, plan.outdim), dtype=torch.float32, device=x.device)
    nbytes = fc_workspace(plan, N, H)
    if ws is None:
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    elif ws.numel() < nbytes:
        raise ValueError(f"workspace too small: {ws.numel()} < {nbytes} bytes")
    g = graph.cstruct()
    _check(lib().tp_conv_forward_fc(plan.handle, ctypes.byref(g), _ptr(x), _ptr(Y), _ptr(R), H,
                                    _ptr(Theta), _ptr(out), _ptr(ws), ws.numel(), _stream(x.device)))
    return out


def gaunt_dims(plan):
    """(outdim, weights per edge, grid points) of the Gaunt product of this plan"""
    o, w, q = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib().tp_conv_gaunt_dims(plan.handle, ctypes.byref(o), ctypes.byref(w), ctypes.byref(q)))
    return o.value, w.value, q.value


def forward_gaunt(plan, graph, x, Y, w, out=None):
    """out [N, U (lmax_out+1)^2] of the Gaunt (spherical-grid) convolution:
    receiver-sorted Y [E, ysh] and filter weights w [E, lmax_sh+1, U] (or [E, wdim])."""
    torch = _torch()
    N, E = graph.n_nodes, graph.n_edges
    outdim, wdim, _ = gaunt_dims(plan)
    _need(x, "x", torch.float32, (N, plan.xdim))
    _need(Y, "Y", torch.float32, (E, plan.ysh))
    if w.dim() == 3:
        _need(w, "w", torch.float32, (E, plan.lmax_sh + 1, plan.mul))
    else:
        _need(w, "w", torch.float32, (E, wdim))
    if out is None:
        out = torch.empty((N, outdim), dtype=torch.float32, device=x.device)
    _need(out, "out", torch.float32, (N, outdim))
    g = graph.cstruct()
    _check(lib().tp_conv_forward_gaunt(plan.handle, ctypes.byref(g), _ptr(x), _ptr(Y), _ptr(w),
                                       _ptr(out), _stream(x.device)))
    return out


def backward_gaunt(plan, graph, x, Y, w, grad_out, want=("x", "Y", "w"), outs=None):
    """(grad_x, grad_Y, grad_w) of the Gaunt convolution for grad_out [N, outdim];
    entries not in ``want`` are None (skipped on the device).  grad_w has w's shape."""
    torch = _torch()
    N, E = graph.n_nodes, graph.n_edges
    outdim, wdim, _ = gaunt_dims(plan)
    _need(x, "x", torch.float32, (N, plan.xdim))
    _need(Y, "Y", torch.float32, (E, plan.ysh))
    _need(w, "w", torch.float32, tuple(w.shape))
    if w.numel() != E * wdim:
        raise ValueError(f"w has {w.numel()} elements, expected {E * wdim}")
    _need(grad_out, "grad_out", torch.float32, (N, outdim))
    if outs is None:
        outs = (torch.empty_like(x) if "x" in want else None,
                torch.empty_like(Y) if "Y" in want else None,
                torch.empty_like(w) if "w" in want else None)
    gx, gY, gw = outs
    g = graph.cstruct()
    _check(lib().tp_conv_backward_gaunt(plan.handle, ctypes.byref(g), _ptr(x), _ptr(Y), _ptr(w),
                                        _ptr(grad_out), _ptr(gx), _ptr(gY), _ptr(gw), _stream(x.device)))
    return gx, gY, gw


def gaunt_double_workspace(plan, n_nodes, n_edges):
    """bytes of workspace double_backward_gaunt needs"""
    b = ctypes.c_size_t()
    _check(lib().tp_conv_gaunt_double_workspace(plan.handle, n_nodes, n_edges, ctypes.byref(b)))
    return b.value


def double_backward_gaunt(plan, graph, x, Y, w, grad_out, gg_x=None, gg_Y=None, gg_w=None,
                          want=("x", "Y", "w", "g"), ws=None):
    """(d_x, d_Y, d_w, d_grad_out): gradients of <gg_x, grad_x> + <gg_Y, grad_Y> +
    <gg_w, grad_w> (the outputs of backward_gaunt) with respect to its inputs;
    missing cotangents are zero, outputs not in ``want`` are None."""
    torch = _torch()
    N, E = graph.n_nodes, graph.n_edges
    outdim, wdim, _ = gaunt_dims(plan)
    _need(x, "x", torch.float32, (N, plan.xdim))
    _need(Y, "Y", torch.float32, (E, plan.ysh))
    _need(w, "w", torch.float32, tuple(w.shape))
    if w.numel() != E * wdim:
        raise ValueError(f"w has {w.numel()} elements, expected {E * wdim}")
    _need(grad_out, "grad_out", torch.float32, (N, outdim))
    for t, like, name in ((gg_x, x, "gg_x"), (gg_Y, Y, "gg_Y"), (gg_w, w, "gg_w")):
        if t is not None:
            _need(t, name, torch.float32, tuple(like.shape))
    nbytes = gaunt_double_workspace(plan, N, E)
    if ws is None:
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    elif ws.numel() < nbytes:
        raise ValueError(f"workspace too small: {ws.numel()} < {nbytes} bytes")
    mk = lambda name, like: torch.empty_like(like) if name in want else None
    dx, dY, dw, dg = mk("x", x), mk("Y", Y), mk("w", w), mk("g", grad_out)
    g = graph.cstruct()
    _check(lib().tp_conv_double_backward_gaunt(plan.handle, ctypes.byref(g), _ptr(x), _ptr(Y), _ptr(w),
                                               _ptr(grad_out), _ptr(gg_x), _ptr(gg_Y), _ptr(gg_w), _ptr(dx),
                                               _ptr(dY), _ptr(dw), _ptr(dg), _ptr(ws), ws.numel(),
                                               _stream(x.device)))
    return dx, dY, dw, dg


def fc_backward_workspace(plan, n_nodes, n_radial):
    """bytes of the node-sized states backward_fc needs"""
    b = ctypes.c_size_t()
    _check(lib().tp_conv_fc_backward_workspace(plan.handle, n_nodes, n_radial, ctypes.byref(b)))
    return b.value


def fc_double_workspace(plan, n_nodes, n_edges, n_radial):
    """bytes of workspace double_backward_fc needs"""
    b = ctypes.c_size_t()
    _check(lib().tp_conv_fc_double_workspace(plan.handle, n_nodes, n_edges, n_radial, ctypes.byref(b)))
    return b.value


def double_backward_fc(plan, graph, x, Y, R, Theta, grad_out, gg_x=None, gg_Y=None, gg_R=None, gg_Theta=None,
                       want=("x", "Y", "R", "Theta", "g"), ws=None):
    """(d_x, d_Y, d_R, d_Theta, d_grad_out): gradients of <gg_x, grad_x> + <gg_Y, grad_Y>
    + <gg_R, grad_R> + <gg_Theta, grad_Theta> (the outputs of backward_fc) with respect
    to its inputs; missing cotangents are zero, outputs not in ``want`` are None."""
    torch = _torch()
    N, E = graph.n_nodes, graph.n_edges
    H = R.shape[1]
    _need(x, "x", torch.float32, (N, plan.xdim))
    _need(Y, "Y", torch.float32, (E, plan.ysh))
    _need(R, "R", torch.float32, (E, H))
    _need(Theta, "Theta", torch.float32, (H, plan.n_paths, plan.mul, plan.mul))
    _need(grad_out, "grad_out", torch.float32, (N, plan.outdim))
    for t, like, name in ((gg_x, x, "gg_x"), (gg_Y, Y, "gg_Y"), (gg_R, R, "gg_R"), (gg_Theta, Theta, "gg_Theta")):
        if t is not None:
            _need(t, name, torch.float32, tuple(like.shape))
    nbytes = fc_double_workspace(plan, N, E, H)
    if ws is None:
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    elif ws.numel() < nbytes:
        raise ValueError(f"workspace too small: {ws.numel()} < {nbytes} bytes")
    mk = lambda name, like: torch.empty_like(like) if name in want else None
    dx, dY, dR, dT, dg = mk("x", x), mk("Y", Y), mk("R", R), mk("Theta", Theta), mk("g", grad_out)
    g = graph.cstruct()
    _check(lib().tp_conv_double_backward_fc(plan.handle, ctypes.byref(g), _ptr(x), _ptr(Y), _ptr(R), H,
                                            _ptr(Theta), _ptr(grad_out), _ptr(gg_x), _ptr(gg_Y), _ptr(gg_R),
                                            _ptr(gg_Theta), _ptr(dx), _ptr(dY), _ptr(dR), _ptr(dT), _ptr(dg),
                                            _ptr(ws), ws.numel(), _stream(x.device)))
    return dx, dY, dR, dT, dg


def backward_fc(plan, graph, x, Y, R, Theta, grad_out, want=("x", "Y", "R", "Theta"), ws=None, outs=None,
                state_saved=False):
    """(grad_x, grad_Y, grad_R, grad_Theta) of the fully connected convolution;
    entries not in ``want`` (or None in ``outs``) are None (skipped on the device).
    ``state_saved``: ``ws`` is the workspace ``forward_fc`` was given for the
    same graph and inputs and still holds its state (read instead of recomputed)."""
    torch = _torch()
    N, E = graph.n_nodes, graph.n_edges
    H = R.shape[1]
    _need(x, "x", torch.float32, (N, plan.xdim))
    _need(Y, "Y", torch.float32, (E, plan.ysh))
    _need(R, "R", torch.float32, (E, H))
    _need(Theta, "Theta", torch.float32, (H, plan.n_paths, plan.mul, plan.mul))
    _need(grad_out, "grad_out", torch.float32, (N, plan.outdim))
    nbytes = fc_backward_workspace(plan, N, H)
    if ws is None:
        if state_saved:
            raise ValueError("state_saved needs the workspace the forward wrote")
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    elif ws.numel() < nbytes:
        raise ValueError(f"workspace too small: {ws.numel()} < {nbytes} bytes")
    if outs is None:
        outs = (torch.empty_like(x) if "x" in want else None,
                torch.empty_like(Y) if "Y" in want else None,
                torch.empty_like(R) if "R" in want else None,
                torch.empty_like(Theta) if "Theta" in want else None)
    gx, gY, gR, gT = outs
    g = graph.cstruct()
    _check(lib().tp_conv_backward_fc(plan.handle, ctypes.byref(g), _ptr(x), _ptr(Y), _ptr(R), H, _ptr(Theta),
                                     _ptr(grad_out), _ptr(gx), _ptr(gY), _ptr(gR), _ptr(gT),
                                     TP_FC_STATE_SAVED if state_saved else 0, _ptr(ws), ws.numel(),
                                     _stream(x.device)))
    return gx, gY, gR, gT


def uvw_forward(plan, Wmix, x_in, out=None):
    """Per-output-irrep U x U channel mix of node rows x_in [N, outdim]."""
    torch = _torch()
    N = x_in.shape[0]
    _need(x_in, "in", torch.float32, (N, plan.outdim))
    K = len(plan.out_irreps.split("+"))
    _need(Wmix, "Wmix", torch.float32, (K, plan.mul, plan.mul))
    if out is None:
        out = torch.empty_like(x_in)
    _check(lib().tp_conv_uvw_forward(plan.handle, N, _ptr(Wmix), _ptr(x_in), _ptr(out),
                                     _stream(x_in.device)))
    return out


def uvw_backward(plan, Wmix, x_in, grad_out, want=("in", "W")):
    """(grad_in, grad_Wmix) of the channel mix; entries not in ``want`` are None."""
    torch = _torch()
    N = grad_out.shape[0]
    _need(grad_out, "grad_out", torch.float32, (N, plan.outdim))
    K = len(plan.out_irreps.split("+"))
    _need(Wmix, "Wmix", torch.float32, (K, plan.mul, plan.mul))
    gi = torch.empty_like(grad_out) if "in" in want else None
    gW = torch.empty_like(Wmix) if "W" in want else None
    ws, nbytes = None, 0
    if gW is not None:
        _need(x_in, "in", torch.float32, (N, plan.outdim))
        b = ctypes.c_size_t()
        _check(lib().tp_conv_uvw_workspace(plan.handle, ctypes.byref(b)))
        nbytes = b.value
        ws = torch.empty(nbytes, dtype=torch.uint8, device=grad_out.device)
    _check(lib().tp_conv_uvw_backward(plan.handle, N, _ptr(Wmix), _ptr(x_in), _ptr(grad_out),
                                      _ptr(gi), _ptr(gW), _ptr(ws), nbytes,
                                      _stream(grad_out.device)))
    return gi, gW


def forward_radial(plan, graph, x, Y, r_len, W1, W2, Wmix=None, out=None, out_pre=None):
    """(out, out_pre) of the radial-weight convolution; out_pre is None without a mix."""
    torch = _torch()
    N, E = graph.n_nodes, graph.n_edges
    nb, nh, _ = plan.radial
    _need(x, "x", torch.float32, (N, plan.xdim))
    _need(Y, "Y", torch.float32, (E, plan.ysh))
    _need(r_len, "r_len", torch.float32, (E,))
    _need(W1, "W1", torch.float32, (nb, nh))
    _need(W2, "W2", torch.float32, (nh, plan.n_paths * plan.mul))
    f32 = dict(dtype=torch.float32, device=x.device)
    if out is None:
        out = torch.empty((N, plan.outdim), **f32)
    if Wmix is not None and out_pre is None:
        out_pre = torch.empty((N, plan.outdim), **f32)
    g = graph.cstruct()
    _check(lib().tp_conv_forward_radial(plan.handle, ctypes.byref(g), _ptr(x), _ptr(Y),
                                        _ptr(r_len), _ptr(W1), _ptr(W2), _ptr(Wmix),
                                        _ptr(out_pre) if Wmix is not None else None, _ptr(out),
                                        _stream(x.device)))
    return out, (out_pre if Wmix is not None else None)


def backward_radial(plan, graph, x, Y, r_len, W1, W2, grad_out, Wmix=None, out_pre=None,
                    want=("x", "Y", "W1", "W2", "Wmix"), outs=None, ws=None):
    """(grad_x, grad_Y, grad_W1, grad_W2, grad_Wmix, grad_rlen) of the radial-weight
    convolution (grad_Y, grad_rlen receiver-sorted); entries not in ``want`` (names
    x, Y, W1, W2, Wmix, rlen) and grad_Wmix without a mix are None.  ``outs`` (a
    dict name -> tensor) and ``ws`` (uint8, at least radial_workspace bytes)
    supply preallocated buffers."""
    torch = _torch()
    N, E = graph.n_nodes, graph.n_edges
    nb, nh, _ = plan.radial
    _need(x, "x", torch.float32, (N, plan.xdim))
    _need(Y, "Y", torch.float32, (E, plan.ysh))
    _need(r_len, "r_len", torch.float32, (E,))
    _need(W1, "W1", torch.float32, (nb, nh))
    _need(W2, "W2", torch.float32, (nh, plan.n_paths * plan.mul))
    _need(grad_out, "grad_out", torch.float32, (N, plan.outdim))
    if Wmix is not None:
        K = len(plan.out_irreps.split("+"))
        _need(Wmix, "Wmix", torch.float32, (K, plan.mul, plan.mul))
        if "Wmix" in want:
            _need(out_pre, "out_pre", torch.float32, (N, plan.outdim))
    outs = outs or {}

    def buf(name, like):
        if name not in want or like is None:
            return None
        t = outs.get(name)
        if t is None:
            return torch.empty_like(like)
        _need(t, "grad_" + name, torch.float32, tuple(like.shape))
        return t
    gx, gY, gW1, gW2 = buf("x", x), buf("Y", Y), buf("W1", W1), buf("W2", W2)
    gWm = buf("Wmix", Wmix)
    grl = buf("rlen", r_len)
    nbytes = radial_workspace(plan, N, Wmix is not None)
    if ws is None:
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    elif ws.numel() < nbytes:
        raise ValueError(f"workspace too small: {ws.numel()} < {nbytes} bytes")
    g = graph.cstruct()
    _check(lib().tp_conv_backward_radial(plan.handle, ctypes.byref(g), _ptr(x), _ptr(Y), _ptr(r_len),
                                         _ptr(W1), _ptr(W2), _ptr(Wmix),
                                         _ptr(out_pre) if gWm is not None else None, _ptr(grad_out),
                                         _ptr(gx), _ptr(gY), _ptr(grl), _ptr(gW1), _ptr(gW2),
                                         _ptr(gWm), _ptr(ws), ws.numel(), _stream(x.device)))
    return gx, gY, gW1, gW2, gWm, grl


def forward_radial_r(plan, graph, x, r, W1, W2, Wmix=None, out=None, out_pre=None):
    """forward_radial from the edge vectors r [E, 3] (receiver-sorted): harmonics
    and lengths evaluated on chip."""
    torch = _torch()
    N, E = graph.n_nodes, graph.n_edges
    nb, nh, _ = plan.radial
    _need(x, "x", torch.float32, (N, plan.xdim))
    _need(r, "r", torch.float32, (E, 3))
    _need(W1, "W1", torch.float32, (nb, nh))
    _need(W2, "W2", torch.float32, (nh, plan.n_paths * plan.mul))
    f32 = dict(dtype=torch.float32, device=x.device)
    if out is None:
        out = torch.empty((N, plan.outdim), **f32)
    if Wmix is not None and out_pre is None:
        out_pre = torch.empty((N, plan.outdim), **f32)
    g = graph.cstruct()
    _check(lib().tp_conv_forward_radial_r(plan.handle, ctypes.byref(g), _ptr(x), _ptr(r), _ptr(W1),
                                          _ptr(W2), _ptr(Wmix),
                                          _ptr(out_pre) if Wmix is not None else None, _ptr(out),
                                          _stream(x.device)))
    return out, (out_pre if Wmix is not None else None)


def backward_radial_r(plan, graph, x, r, W1, W2, grad_out, Wmix=None, out_pre=None,
                      want=("x", "r", "W1", "W2", "Wmix"), outs=None, ws=None):
    """(grad_x, grad_r, grad_W1, grad_W2, grad_Wmix) of forward_radial_r; grad_r [E, 3]
    (receiver-sorted) is the gradient with respect to the edge vectors through the
    harmonics and the lengths.  Entries not in ``want`` and grad_Wmix without a mix
    are None."""
    torch = _torch()
    N, E = graph.n_nodes, graph.n_edges
    nb, nh, _ = plan.radial
    _need(x, "x", torch.float32, (N, plan.xdim))
    _need(r, "r", torch.float32, (E, 3))
    _need(W1, "W1", torch.float32, (nb, nh))
    _need(W2, "W2", torch.float32, (nh, plan.n_paths * plan.mul))
    _need(grad_out, "grad_out", torch.float32, (N, plan.outdim))
    if Wmix is not None:
        K = len(plan.out_irreps.split("+"))
        _need(Wmix, "Wmix", torch.float32, (K, plan.mul, plan.mul))
        if "Wmix" in want:
            _need(out_pre, "out_pre", torch.float32, (N, plan.outdim))
    outs = outs or {}

    def buf(name, like):
        if name not in want or like is None:
            return None
        t = outs.get(name)
        if t is None:
            return torch.empty_like(like)
        _need(t, "grad_" + name, torch.float32, tuple(like.shape))
        return t
    gx, gr, gW1, gW2 = buf("x", x), buf("r", r), buf("W1", W1), buf("W2", W2)
    gWm = buf("Wmix", Wmix)
    nbytes = radial_workspace(plan, N, Wmix is not None)
    if ws is None:
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    elif ws.numel() < nbytes:
        raise ValueError(f"workspace too small: {ws.numel()} < {nbytes} bytes")
    g = graph.cstruct()
    _check(lib().tp_conv_backward_radial_r(plan.handle, ctypes.byref(g), _ptr(x), _ptr(r), _ptr(W1),
                                           _ptr(W2), _ptr(Wmix),
                                           _ptr(out_pre) if gWm is not None else None, _ptr(grad_out),
                                           _ptr(gx), _ptr(gr), _ptr(gW1), _ptr(gW2), _ptr(gWm), _ptr(ws),
                                           ws.numel(), _stream(x.device)))
    return gx, gr, gW1, gW2, gWm


def double_backward_radial(plan, graph, x, Y, r_len, W1, W2, grad_out, Wmix=None, gg_x=None, gg_Y=None,
                           gg_rlen=None, want=("x", "Y", "rlen", "W1", "W2", "Wmix", "g"), outs=None,
                           ws=None):
    """(d_x, d_Y, d_rlen, d_W1, d_W2, d_Wmix, d_grad_out): gradients of
    <gg_x, grad_x> + <gg_Y, grad_Y> + <gg_rlen, grad_rlen> (the outputs of
    backward_radial) with respect to its inputs; missing cotangents are zero,
    outputs not in ``want`` (and d_Wmix without a mix) are None.  ``outs`` (a
    dict name -> tensor) and ``ws`` supply preallocated buffers."""
    torch = _torch()
    N, E = graph.n_nodes, graph.n_edges
    nb, nh, _ = plan.radial
    _need(x, "x", torch.float32, (N, plan.xdim))
    _need(Y, "Y", torch.float32, (E, plan.ysh))
    _need(r_len, "r_len", torch.float32, (E,))
    _need(W1, "W1", torch.float32, (nb, nh))
    _need(W2, "W2", torch.float32, (nh, plan.n_paths * plan.mul))
    _need(grad_out, "grad_out", torch.float32, (N, plan.outdim))
    if Wmix is not None:
        K = len(plan.out_irreps.split("+"))
        _need(Wmix, "Wmix", torch.float32, (K, plan.mul, plan.mul))
    for t, name, shape in ((gg_x, "gg_x", (N, plan.xdim)), (gg_Y, "gg_Y", (E, plan.ysh)),
                           (gg_rlen, "gg_rlen", (E,))):
        if t is not None:
            _need(t, name, torch.float32, shape)
    outs = outs or {}

    def buf(name, like):
        if name not in want or like is None:
            return None
        t = outs.get(name)
        if t is None:
            return torch.empty_like(like)
        _need(t, "d_" + name, torch.float32, tuple(like.shape))
        return t
    dx, dY, drl = buf("x", x), buf("Y", Y), buf("rlen", r_len)
    dW1, dW2, dWm, dg = buf("W1", W1), buf("W2", W2), buf("Wmix", Wmix), buf("g", grad_out)
    nbytes = radial_double_workspace(plan, N, Wmix is not None)
    if ws is None:
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    elif ws.numel() < nbytes:
        raise ValueError(f"workspace too small: {ws.numel()} < {nbytes} bytes")
    g = graph.cstruct()
    _check(lib().tp_conv_double_backward_radial(
        plan.handle, ctypes.byref(g), _ptr(x), _ptr(Y), _ptr(r_len), _ptr(W1), _ptr(W2), _ptr(Wmix),
        _ptr(grad_out), _ptr(gg_x), _ptr(gg_Y), _ptr(gg_rlen), _ptr(dx), _ptr(dY), _ptr(drl), _ptr(dW1),
        _ptr(dW2), _ptr(dWm), _ptr(dg), _ptr(ws), ws.numel(), _stream(x.device)))
    return dx, dY, drl, dW1, dW2, dWm, dg


def radial_double_workspace(plan, n_nodes, with_mix):
    """bytes of workspace double_backward_radial needs"""
    b = ctypes.c_size_t()
    _check(lib().tp_conv_radial_double_workspace(plan.handle, n_nodes, int(bool(with_mix)), ctypes.byref(b)))
    return b.value


def radial_workspace(plan, n_nodes, with_mix):
    """bytes of workspace backward_radial needs"""
    b = ctypes.c_size_t()
    _check(lib().tp_conv_radial_workspace(plan.handle, n_nodes, int(bool(with_mix)), ctypes.byref(b)))
    return b.value
