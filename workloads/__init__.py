"""Seeded synthetic workloads for the tensor-product convolution.

This module draws inputs only: graphs, edge vectors, node features, edge
weights, radial-network parameters and upstream gradients.  It holds none of
the method's arithmetic (no harmonics, CG, paths or convolution) and imports
neither the oracle nor the GPU package; both sides receive the same arrays.

Shapes and distributions follow the workloads the pages measure on or
describe: the 1,536-atom / 46,080-edge molecular graph of "Accelerating Tensor
Products in E(3)-Equivariant Graph Neural Networks" (Abstract), variable
degree (5 to 30 neighbours) and hub atoms of "The GPU Workload That Rewrites
Molecular Physics" (section "What Makes MLFF Workloads Structurally
Different"), and the edge-scaling regime of "Sobek: Streaming Equivariant
Tensor Product Convolutions" (Abstract).  The pages' own graphs are not
available; these synthetic graphs stand in for them.

Every array is drawn in float64 and rounded to float32 once; the oracle is
then fed the float32 values (upcast), so input rounding is never counted as
kernel error.  Edge lists are shuffled so that grouping by receiver is real
work.  Draw order: graph, shuffle, edge vectors, x, weights, gradient.
"""
from dataclasses import dataclass

import numpy as np

# name -> (irreps, lmax_sh, lmax_out, default n_nodes, graph kind, weight kind)
CONFIGS = {
    "tiny":   dict(irreps="8x0e+8x1o", lmax_sh=2, lmax_out=2, n_nodes=32,
                   graph="box", w_std="one", modes=("fwd", "fwd+bwd")),
    "mid":    dict(irreps="32x0e+32x1o+32x2e", lmax_sh=2, lmax_out=2, n_nodes=1536,
                   graph="fixed30", w_std="paths", modes=("fwd", "fwd+bwd")),
    "lmax3":  dict(irreps="64x0e+64x1o+64x2e+64x3o", lmax_sh=3, lmax_out=3, n_nodes=4096,
                   graph="uniform5_30", w_std="paths", modes=("fwd",)),
    "zipf":   dict(irreps="64x0e+64x1o+64x2e+64x3o", lmax_sh=3, lmax_out=3, n_nodes=32768,
                   graph="zipf", w_std="paths", modes=("fwd", "fwd+bwd")),
    "stream": dict(irreps="128x0e+128x1o+128x2e", lmax_sh=2, lmax_out=2, n_nodes=100000,
                   graph="fixed30", w_std="radial", modes=("fwd", "fwd+bwd"),
                   n_basis=8, hidden=64, r_cut=5.0),
    # the lmax-3 graph and features with radial-network weights (the streaming
    # layer at the lmax-3 width; the pages give no such configuration)
    "lmax3_radial": dict(irreps="64x0e+64x1o+64x2e+64x3o", lmax_sh=3, lmax_out=3, n_nodes=4096,
                         graph="uniform5_30", w_std="radial", modes=("fwd", "fwd+bwd"),
                         n_basis=8, hidden=64, r_cut=5.0),
}

BOX = 8.0          # periodic cube edge (Angstrom) of the tiny workload
CUTOFF = 4.0       # neighbour cutoff of the tiny workload
LEN_LO, LEN_HI = 0.8, 5.0   # edge-length range of the other workloads
ZIPF_S, ZIPF_CAP = 1.5, 256


@dataclass
class Workload:
    name: str
    irreps: str
    lmax_sh: int
    lmax_out: int
    n_nodes: int
    src: np.ndarray      # int32 [E], original (shuffled) edge order
    dst: np.ndarray      # int32 [E]
    r: np.ndarray        # float32 [E, 3], sender minus receiver
    x: np.ndarray        # float32 [N, xdim]
    w: np.ndarray = None       # float32 [E, P, U] (direct weights)
    W1: np.ndarray = None      # float32 [n_basis, hidden] (radial weights)
    W2: np.ndarray = None      # float32 [hidden, P*U]
    Wmix: np.ndarray = None    # float32 [K_out, U, U]
    g: np.ndarray = None       # float32 [N, outdim]
    n_basis: int = 0
    r_cut: float = 0.0

    @property
    def n_edges(self):
        return int(self.src.shape[0])

    @property
    def r_len(self):
        return np.linalg.norm(self.r.astype(np.float64), axis=1).astype(np.float32)


def _f32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))


def _distinct_senders(rng, n_nodes, deg):
    """Senders for receiver-major edges: deg[i] distinct senders j != i, uniform."""
    dst = np.repeat(np.arange(n_nodes, dtype=np.int64), deg)
    src = rng.integers(0, n_nodes - 1, size=dst.shape[0])
    src += src >= dst
    while True:
        order = np.lexsort((src, dst))
        ks, kd = src[order], dst[order]
        dup = np.zeros(len(order), dtype=bool)
        dup[1:] = (ks[1:] == ks[:-1]) & (kd[1:] == kd[:-1])
        if not dup.any():
            break
        idx = order[dup]
        s = rng.integers(0, n_nodes - 1, size=idx.shape[0])
        src[idx] = s + (s >= dst[idx])
    return src, dst


def _graph(rng, kind, n_nodes):
    """Returns (src, dst, r) in receiver-major order, before the shuffle."""
    if kind == "box":
        pos = rng.uniform(0.0, BOX, size=(n_nodes, 3))
        d = pos[None, :, :] - pos[:, None, :]          # d[i, j] = pos[j] - pos[i]
        d -= BOX * np.round(d / BOX)                    # minimum image
        dist = np.linalg.norm(d, axis=2)
        mask = (dist < CUTOFF) & ~np.eye(n_nodes, dtype=bool)
        dst, src = np.nonzero(mask)                     # receiver-major
        return src, dst, d[dst, src]
    if kind == "fixed30":
        deg = np.full(n_nodes, min(30, n_nodes - 1), dtype=np.int64)
    elif kind == "uniform5_30":
        deg = rng.integers(5, 31, size=n_nodes)
        deg = np.minimum(deg, n_nodes - 1)
    elif kind == "zipf":
        deg = np.minimum(rng.zipf(ZIPF_S, size=n_nodes), min(ZIPF_CAP, n_nodes - 1))
    else:
        raise ValueError(kind)
    src, dst = _distinct_senders(rng, n_nodes, deg)
    return src, dst, None


def _directions(rng, n):
    v = rng.normal(size=(n, 3))
    v /= np.linalg.norm(v, axis=1, keepdims=True)
    return v * rng.uniform(LEN_LO, LEN_HI, size=(n, 1))


def make_workload(name, dims, seed=0, n_nodes=None, graph_only=False):
    """Draw one workload.

    ``dims`` gives the sizes the plan fixes: xdim, n_paths, U, outdim and
    n_out_irreps (the generator does not enumerate paths itself).  ``n_nodes``
    overrides the configuration's atom count for reduced-size parity runs.
    ``graph_only`` stops after the edge vectors (the same graph and vectors
    as a full draw, since those are drawn first).
    """
    cfg = CONFIGS[name]
    n = int(n_nodes or cfg["n_nodes"])
    rng = np.random.default_rng(seed)
    src, dst, r = _graph(rng, cfg["graph"], n)
    shuffle = rng.permutation(len(src))
    src, dst = src[shuffle], dst[shuffle]
    r = r[shuffle] if r is not None else _directions(rng, len(src))
    if graph_only:
        return Workload(name=name, irreps=cfg["irreps"], lmax_sh=cfg["lmax_sh"],
                        lmax_out=cfg["lmax_out"], n_nodes=n, src=src.astype(np.int32),
                        dst=dst.astype(np.int32), r=_f32(r), x=None)
    x = rng.normal(size=(n, dims["xdim"]))
    wl = Workload(name=name, irreps=cfg["irreps"], lmax_sh=cfg["lmax_sh"],
                  lmax_out=cfg["lmax_out"], n_nodes=n,
                  src=src.astype(np.int32), dst=dst.astype(np.int32),
                  r=_f32(r), x=_f32(x))
    P, U = dims["n_paths"], dims["U"]
    if cfg["w_std"] == "radial":
        nb, hid = cfg["n_basis"], cfg["hidden"]
        wl.W1 = _f32(rng.normal(size=(nb, hid)) / np.sqrt(nb))
        wl.W2 = _f32(rng.normal(size=(hid, P * U)) / np.sqrt(hid))
        wl.Wmix = _f32(rng.normal(size=(dims["n_out_irreps"], U, U)) / np.sqrt(U))
        wl.n_basis, wl.r_cut = nb, cfg["r_cut"]
    else:
        std = 1.0 if cfg["w_std"] == "one" else 1.0 / np.sqrt(P)
        wl.w = _f32(rng.normal(size=(len(src), P, U)) * std)
    wl.g = _f32(rng.normal(size=(n, dims["outdim"])))
    return wl


def make_fc_inputs(n_edges, n_paths, U, H=8, seed=0):
    """Radial features R [E, H] (edge order of the workload) and channel-mixing
    parameters Theta [H, P, U, U] of the fully connected per-edge-weight layer:
    R ~ N(0, 1), Theta ~ N(0, 1/(H U)), float64 draws rounded to float32."""
    rng = np.random.default_rng(seed + 17)
    R = _f32(rng.normal(size=(n_edges, H)))
    Th = _f32(rng.normal(size=(H, n_paths, U, U)) / np.sqrt(H * U))
    return R, Th


def make_gaunt_weights(n_edges, lmax_sh, U, seed=0):
    """Per-edge filter weights of the Gaunt (spherical-grid) convolution,
    w [E, lmax_sh+1, U] (one weight per edge, filter degree and channel),
    w ~ N(0, 1/(lmax_sh+1)) drawn in float64 and rounded to float32."""
    rng = np.random.default_rng(seed + 29)
    return _f32(rng.normal(size=(n_edges, lmax_sh + 1, U)) / np.sqrt(lmax_sh + 1))
