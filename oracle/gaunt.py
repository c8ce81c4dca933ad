"""The Gaunt (spherical-grid) tensor-product convolution: an explicitly
different operator from the Clebsch-Gordan convolution of ``conv.py``.

Test infrastructure only (see ``oracle/__init__.py``).

"The Price of Freedom: Exploring Expressivity and Runtime Tradeoffs in
Equivariant Tensor Products" (ICML 2025, Abstract) sets the Gaunt tensor
product apart from the full CG product: a different operation, cheaper and
less expressive, which that page evaluates directly on a spherical grid.  The
page prints no formula; the readings taken here are:

* per channel u, a node feature with degrees l1 (natural parity, one
  multiplicity U) is the signal f_{j,u}(s) = sum_{l1,m} x[j,l1,u,m] Y_{l1 m}(s)
  on the unit sphere, and an edge carries the filter
  g_{e,u}(s) = sum_{l2 <= lmax_sh} w[e,l2,u] sum_m Y_e[l2,m] Y_{l2 m}(s)
  (its harmonics, weighted per degree and channel -- the weights must factor
  per degree for the grid evaluation to exist);
* the Gaunt product is the pointwise product f g expanded again in the same
  harmonics up to degree lmax_out; with component normalisation
  (1/4pi) int Y_a Y_b dOmega = delta_ab, so coefficient c is
  (1/4pi) int f g Y_c dOmega;
* out[i, l3, u, m3] = sum_{e = (j -> i)} coefficient (l3, m3) of f_{j,u} g_{e,u}.
  Output irreps are l3 = 0..lmax_out with parity (-1)^l3 (the product of
  natural-parity signals has natural parity), each block [U][2l3+1].

Written out, out = sum_e sum_{l1,l2} w[e,l2,u] sum_{a,b} G[a,b,c] x[j,l1,u,a]
Y_e[l2,b] with the Gaunt coefficients G[a,b,c] = (1/4pi) int Y_a Y_b Y_c.
G vanishes unless l1 + l2 + l3 is even and the triangle rule holds, so the
antisymmetric couplings of the CG product (the cross product 1 x 1 -> 1) are
absent: the loss of expressivity the page measures.

This module computes the written-out form: G by an exact product quadrature
(a library Gauss-Legendre rule in cos(theta) times equispaced azimuths, exact
for polynomials of the total degree), then per-edge messages summed into
receivers with ``np.add.at``.
"""
from dataclasses import dataclass, field

import numpy as np

from .irreps import parse_irreps
from .sh import sh_real

CHUNK = 8192


def sphere_quadrature(degree):
    """Points [Q, 3] on the unit sphere and weights [Q] (summing to 4 pi) that
    integrate every polynomial of total degree <= ``degree`` exactly: Gauss-
    Legendre in cos(theta) with ceil((degree+1)/2) nodes, times degree+1
    equispaced azimuths (exact for e^{i m phi}, |m| <= degree)."""
    n_t = (degree + 2) // 2
    n_p = degree + 1
    ct, wt = np.polynomial.legendre.leggauss(max(n_t, 1))
    phi = 2 * np.pi * np.arange(n_p) / n_p
    st = np.sqrt(1.0 - ct ** 2)
    pts = np.stack([np.outer(st, np.cos(phi)), np.outer(st, np.sin(phi)),
                    np.outer(ct, np.ones(n_p))], axis=-1).reshape(-1, 3)
    wts = np.outer(wt, np.full(n_p, 2 * np.pi / n_p)).reshape(-1)
    return pts, wts


def gaunt_coefficients(l1, l2, l3):
    """G[a, b, c] = (1/4pi) int Y_{l1 a} Y_{l2 b} Y_{l3 c} dOmega for the real
    component-normalised harmonics, shape [2l1+1, 2l2+1, 2l3+1].  Rounding
    residue (|G| <= 1e-13) is set to exactly zero."""
    pts, wts = sphere_quadrature(l1 + l2 + l3)
    lm = max(l1, l2, l3)
    Ys = sh_real(lm, pts)
    A = Ys[:, l1 * l1:(l1 + 1) ** 2]
    B = Ys[:, l2 * l2:(l2 + 1) ** 2]
    C = Ys[:, l3 * l3:(l3 + 1) ** 2]
    G = np.einsum("q,qa,qb,qc->abc", wts / (4 * np.pi), A, B, C)
    G[np.abs(G) <= 1e-13] = 0.0
    return G


@dataclass
class GauntPlan:
    """Layout of the Gaunt convolution (readings in the module docstring)."""
    degrees: list             # input degrees l1, string order
    U: int
    lmax_sh: int
    lmax_out: int
    in_offsets: list
    out_offsets: list         # block l3 starts at U * l3^2
    xdim: int
    outdim: int
    ysh: int
    wdim: int                 # weights per edge: (lmax_sh + 1) * U, layout [l2][u]
    G: dict = field(default_factory=dict)   # (l1, l2, l3) -> G, only nonzero triples

    def out_irreps_str(self):
        return "+".join(f"{self.U}x{l}{'e' if l % 2 == 0 else 'o'}"
                        for l in range(self.lmax_out + 1))


def gaunt_plan(irreps_in, lmax_sh, lmax_out):
    irr = parse_irreps(irreps_in) if isinstance(irreps_in, str) else list(irreps_in)
    muls = {m for m, _, _ in irr}
    if len(muls) != 1:
        raise ValueError("one multiplicity shared by all input irreps")
    degs = [l for _, l, _ in irr]
    for _, l, p in irr:
        if p != (-1) ** l:
            raise ValueError("input irreps must have natural parity (-1)^l")
    if len(set(degs)) != len(degs):
        raise ValueError("each input degree at most once (a signal per channel)")
    if lmax_sh < 0 or lmax_out < 0:
        raise ValueError("lmax must be >= 0")
    U = muls.pop()
    in_off, o = [], 0
    for l in degs:
        in_off.append(o)
        o += U * (2 * l + 1)
    gp = GauntPlan(degrees=degs, U=U, lmax_sh=lmax_sh, lmax_out=lmax_out,
                   in_offsets=in_off, out_offsets=[U * l * l for l in range(lmax_out + 1)],
                   xdim=o, outdim=U * (lmax_out + 1) ** 2, ysh=(lmax_sh + 1) ** 2,
                   wdim=(lmax_sh + 1) * U)
    for l1 in degs:
        for l2 in range(lmax_sh + 1):
            for l3 in range(lmax_out + 1):
                if (l1 + l2 + l3) % 2 or l3 < abs(l1 - l2) or l3 > l1 + l2:
                    continue
                gp.G[(l1, l2, l3)] = gaunt_coefficients(l1, l2, l3)
    return gp


def gaunt_conv_fwd(gp, src, dst, n_nodes, x, Y, w):
    """out [n_nodes, outdim] for x [n_nodes, xdim], Y [E, ysh], w [E, lmax_sh+1, U]
    (or [E, wdim]); edge e carries sender src[e] into receiver dst[e]."""
    src = np.asarray(src, dtype=np.int64)
    dst = np.asarray(dst, dtype=np.int64)
    x = np.asarray(x, dtype=np.float64)
    Y = np.asarray(Y, dtype=np.float64)
    E, U = len(src), gp.U
    w = np.asarray(w, dtype=np.float64).reshape(E, gp.lmax_sh + 1, U)
    if x.shape != (n_nodes, gp.xdim) or Y.shape != (E, gp.ysh) or len(dst) != E:
        raise ValueError("shape mismatch")
    if E and (src.min() < 0 or src.max() >= n_nodes or dst.min() < 0 or dst.max() >= n_nodes):
        raise ValueError("node index out of range")
    out = np.zeros((n_nodes, gp.outdim))
    for s in range(0, E, CHUNK):
        e = slice(s, min(E, s + CHUNK))
        n = e.stop - e.start
        xe, Ye, we = x[src[e]], Y[e], w[e]
        msg = np.zeros((n, gp.outdim))
        for (l1, l2, l3), G in gp.G.items():
            i = gp.degrees.index(l1)
            xa = xe[:, gp.in_offsets[i]:gp.in_offsets[i] + U * (2 * l1 + 1)].reshape(n, U, 2 * l1 + 1)
            yb = Ye[:, l2 * l2:(l2 + 1) ** 2]
            t = np.einsum("abc,eua,eb->euc", G, xa, yb, optimize=True) * we[:, l2, :, None]
            o = gp.out_offsets[l3]
            msg[:, o:o + U * (2 * l3 + 1)] += t.reshape(n, U * (2 * l3 + 1))
        np.add.at(out, dst[e], msg)
    return out


def gaunt_conv_bwd(gp, src, dst, n_nodes, x, Y, w, g):
    """Exact adjoint of ``gaunt_conv_fwd`` for the upstream gradient g [n_nodes,
    outdim]: (grad_x [n_nodes, xdim], grad_Y [E, ysh], grad_w [E, lmax_sh+1, U]).
    The forward is linear in each of x, Y and w, so each gradient is the
    forward's coefficient sum with that operand left out."""
    src = np.asarray(src, dtype=np.int64)
    dst = np.asarray(dst, dtype=np.int64)
    x = np.asarray(x, dtype=np.float64)
    Y = np.asarray(Y, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    E, U = len(src), gp.U
    w = np.asarray(w, dtype=np.float64).reshape(E, gp.lmax_sh + 1, U)
    if x.shape != (n_nodes, gp.xdim) or Y.shape != (E, gp.ysh) or g.shape != (n_nodes, gp.outdim):
        raise ValueError("shape mismatch")
    gx = np.zeros_like(x)
    gY = np.zeros_like(Y)
    gw = np.zeros_like(w)
    for s in range(0, E, CHUNK):
        e = slice(s, min(E, s + CHUNK))
        n = e.stop - e.start
        xe, Ye, we, ge = x[src[e]], Y[e], w[e], g[dst[e]]
        gxe = np.zeros((n, gp.xdim))
        for (l1, l2, l3), G in gp.G.items():
            i = gp.degrees.index(l1)
            xs = slice(gp.in_offsets[i], gp.in_offsets[i] + U * (2 * l1 + 1))
            xa = xe[:, xs].reshape(n, U, 2 * l1 + 1)
            yb = Ye[:, l2 * l2:(l2 + 1) ** 2]
            o = gp.out_offsets[l3]
            gc = ge[:, o:o + U * (2 * l3 + 1)].reshape(n, U, 2 * l3 + 1)
            wl = we[:, l2, :]
            # d/dw: sum over a, b, c;  d/dY: sum over u, a, c;  d/dx: sum over b, c
            gw[e, l2, :] += np.einsum("abc,eua,eb,euc->eu", G, xa, yb, gc, optimize=True)
            gY[e, l2 * l2:(l2 + 1) ** 2] += np.einsum("abc,eua,euc,eu->eb", G, xa, gc, wl, optimize=True)
            gxe[:, xs] += np.einsum("abc,eb,euc,eu->eua", G, yb, gc, wl, optimize=True).reshape(n, -1)
        np.add.at(gx, src[e], gxe)
    return gx, gY, gw


def gaunt_conv_double_bwd(gp, src, dst, n_nodes, x, Y, w, g, ggx=None, ggY=None, ggw=None):
    """Second-order backward of the Gaunt convolution.  F(g, x, Y, w) =
    <g, out> is linear in each argument, so for cotangents (ggx, ggY, ggw) of
    the first backward's outputs (None: zero) the loss
    L = <ggx, gx> + <ggY, gY> + <ggw, gw> equals
    F(g, ggx, Y, w) + F(g, x, ggY, w) + F(g, x, Y, ggw), and each of its
    gradients is a sum of first-order results with one operand replaced.
    Returns (dx, dY, dw, dg)."""
    x = np.asarray(x, dtype=np.float64)
    Y = np.asarray(Y, dtype=np.float64)
    E = len(src)
    w = np.asarray(w, dtype=np.float64).reshape(E, gp.lmax_sh + 1, gp.U)
    z = lambda a, like: np.zeros_like(like) if a is None else np.asarray(a, dtype=np.float64).reshape(like.shape)
    ggx, ggY, ggw = z(ggx, x), z(ggY, Y), z(ggw, w)
    args = (gp, src, dst, n_nodes)
    dg = gaunt_conv_fwd(*args, ggx, Y, w) + gaunt_conv_fwd(*args, x, ggY, w) + gaunt_conv_fwd(*args, x, Y, ggw)
    _, gY_x, gw_x = gaunt_conv_bwd(*args, ggx, Y, w, g)      # x -> ggx
    gx_Y, _, gw_Y = gaunt_conv_bwd(*args, x, ggY, w, g)      # Y -> ggY
    gx_w, gY_w, _ = gaunt_conv_bwd(*args, x, Y, ggw, g)      # w -> ggw
    return gx_Y + gx_w, gY_x + gY_w, gw_x + gw_Y, dg
