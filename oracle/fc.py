"""Fully connected per-edge weights ("uvw" on every edge) for the convolution.

Test infrastructure only (see ``oracle/__init__.py``).

The streaming page reassociates radial projection, harmonic coupling and
aggregation for a second operator family whose per-edge weights mix
channels ("Sobek: Streaming Equivariant Tensor Product Convolutions",
Abstract: fully connected multiplicity mixing is preserved).  Reading: the
per-edge weights are a linear map of H radial features R_e,
    W_e[p, u, v] = sum_h R_e[h] Theta[h, p, u, v],
and
    out[i, k, v, c] = sum_{e=(j->i)} sum_{p: k(p)=k} sum_u W_e[p, u, v]
                      sum_{a,b} C_p[a,b,c] x[j, l1(p), u, a] Y_e[l2(p), b].
This module computes it by the plain definition: the per-edge weights and
messages are materialised (in chunks of edges), which the GPU path must not
do.  Output irreps and paths are those of the channel-wise plan; U channels in
and out.
"""
import numpy as np

from .conv import _check, _blocks

FC_CHUNK = 256


def _tp_terms(plan, xe, Ye):
    """per edge, path, channel and output component: sum_ab C x_a Y_b, list over paths
    of arrays [n, U, 2l3+1]"""
    n, U = xe.shape[0], plan.U
    out = []
    for p in range(plan.n_paths):
        xs, ys, _, da, dc = _blocks(plan, p)
        C = plan.cg[p]                                   # [2l1+1, 2l2+1, 2l3+1]
        xp = xe[:, xs].reshape(n, U, da)
        out.append(np.einsum("abc,nua,nb->nuc", C, xp, Ye[:, ys]))
    return out


def fc_conv_fwd(plan, src, dst, n_nodes, x, Y, R, Theta):
    """out [n_nodes, outdim] (float64) of the fully connected per-edge convolution."""
    src, dst, x, Y = _check(plan, src, dst, n_nodes, x, Y)
    R = np.asarray(R, dtype=np.float64)
    Th = np.asarray(Theta, dtype=np.float64)          # [H, P, U, U]
    U = plan.U
    out = np.zeros((n_nodes, plan.outdim))
    for s in range(0, len(src), FC_CHUNK):
        e = slice(s, s + FC_CHUNK)
        W = np.einsum("eh,hpuv->epuv", R[e], Th)       # per-edge weights
        T = _tp_terms(plan, x[src[e]], Y[e])
        msg = np.zeros((W.shape[0], plan.outdim))
        for p in range(plan.n_paths):
            _, _, os_, _, dc = _blocks(plan, p)
            m = np.einsum("euv,euc->evc", W[:, p], T[p])
            msg[:, os_] += m.reshape(W.shape[0], U * dc)
        np.add.at(out, dst[e], msg)
    return out


def fc_conv_bwd(plan, src, dst, n_nodes, x, Y, R, Theta, g):
    """(grad_x, grad_Y, grad_R, grad_Theta) of <g, fc_conv_fwd(...)>."""
    src, dst, x, Y = _check(plan, src, dst, n_nodes, x, Y)
    R = np.asarray(R, dtype=np.float64)
    Th = np.asarray(Theta, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    U = plan.U
    grad_x = np.zeros_like(x)
    grad_Y = np.zeros_like(Y)
    grad_R = np.zeros_like(R)
    grad_Th = np.zeros_like(Th)
    for s in range(0, len(src), FC_CHUNK):
        e = slice(s, s + FC_CHUNK)
        n = len(src[e])
        xe, Ye, ge = x[src[e]], Y[e], g[dst[e]]
        W = np.einsum("eh,hpuv->epuv", R[e], Th)
        T = _tp_terms(plan, xe, Ye)
        gW = np.zeros_like(W)
        gxe = np.zeros_like(xe)
        for p in range(plan.n_paths):
            xs, ys, os_, da, dc = _blocks(plan, p)
            gp = ge[:, os_].reshape(n, U, dc)                          # [e, v, c]
            gW[:, p] = np.einsum("evc,euc->euv", gp, T[p])
            gT = np.einsum("euv,evc->euc", W[:, p], gp)                # d/dT
            C = plan.cg[p]
            xp = xe[:, xs].reshape(n, U, da)
            gxe[:, xs] += np.einsum("abc,euc,eb->eua", C, gT, Ye[:, ys]).reshape(n, U * da)
            grad_Y[s:s + n, ys] += np.einsum("abc,euc,eua->eb", C, gT, xp)
        np.add.at(grad_x, src[e], gxe)
        grad_R[e] = np.einsum("epuv,hpuv->eh", gW, Th)
        grad_Th += np.einsum("eh,epuv->hpuv", R[e], gW)
    return grad_x, grad_Y, grad_R, grad_Th


def fc_conv_double_bwd(plan, src, dst, n_nodes, x, Y, R, Theta, g, ggx=None, ggY=None, ggR=None,
                       ggTheta=None):
    """Second-order backward of the fully connected family ("Sobek", Abstract:
    both operator families through forward, backward and double backward).
    F(g, x, Y, R, Theta) = <g, out> is linear in each argument, so for
    cotangents (ggx, ggY, ggR, ggTheta) of the first backward's outputs (None:
    zero) the loss L = <ggx, gx> + <ggY, gY> + <ggR, gR> + <ggTheta, gTheta>
    equals F(g, ggx, Y, R, Theta) + F(g, x, ggY, R, Theta) + F(g, x, Y, ggR, Theta)
    + F(g, x, Y, R, ggTheta); each gradient of L is a sum of first-order
    results with one operand replaced.  Returns (dx, dY, dR, dTheta, dg)."""
    src, dst, x, Y = _check(plan, src, dst, n_nodes, x, Y)
    R = np.asarray(R, dtype=np.float64)
    Th = np.asarray(Theta, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    z = lambda a, like: np.zeros_like(like) if a is None else np.asarray(a, dtype=np.float64)
    ggx, ggY, ggR, ggTh = z(ggx, x), z(ggY, Y), z(ggR, R), z(ggTheta, Th)
    args = (plan, src, dst, n_nodes)
    dg = (fc_conv_fwd(*args, ggx, Y, R, Th) + fc_conv_fwd(*args, x, ggY, R, Th)
          + fc_conv_fwd(*args, x, Y, ggR, Th) + fc_conv_fwd(*args, x, Y, R, ggTh))
    _, gY_x, gR_x, gT_x = fc_conv_bwd(*args, ggx, Y, R, Th, g)      # x -> ggx
    gx_Y, _, gR_Y, gT_Y = fc_conv_bwd(*args, x, ggY, R, Th, g)      # Y -> ggY
    gx_R, gY_R, _, gT_R = fc_conv_bwd(*args, x, Y, ggR, Th, g)      # R -> ggR
    gx_T, gY_T, gR_T, _ = fc_conv_bwd(*args, x, Y, R, ggTh, g)      # Theta -> ggTheta
    return (gx_Y + gx_R + gx_T, gY_x + gY_R + gY_T, gR_x + gR_Y + gR_T, gT_x + gT_Y + gT_R, dg)
