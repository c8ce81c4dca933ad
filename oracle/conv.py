"""The tensor-product convolution, its adjoint, the radial MLP and the uvw mix.

Test infrastructure only (see ``oracle/__init__.py``).

Definition (the plain reading of the operator the pages describe -- the
NequIP convolution of "Accelerating Tensor Products in E(3)-Equivariant Graph
Neural Networks", Abstract; the edge-conditioned product summed into
receivers of "Sobek: Streaming Equivariant Tensor Product Convolutions",
Abstract; the full CG product of "The Price of Freedom", Abstract):

    out[i, k, u, c] = sum_{e = (j -> i)} sum_{p : k(p) = k} w[e, p, u]
                      * sum_{a, b} C_p[a, b, c] x[j, l1(p), u, a] Y[e, l2(p), b]

Edges are taken in their original order; each edge's message is built in
float64 and added into its receiver with ``np.add.at``.  This is the
conventional schedule (per-edge messages exist in memory); the pages note the
operator itself does not need them (Sobek, Abstract), which is why the GPU
path never builds them.  Edges are processed in chunks only to bound memory.

The backward pass is the exact adjoint of the forward, which is linear in
each of x, w and Y separately.
"""
import numpy as np

CHUNK = 16384


def _blocks(plan, p):
    i, l1, l2, l3, k = plan.paths[p]
    U = plan.U
    xs = slice(plan.in_offsets[i], plan.in_offsets[i] + U * (2 * l1 + 1))
    ys = plan.sh_slice(l2)
    os_ = slice(plan.out_offsets[k], plan.out_offsets[k] + U * (2 * l3 + 1))
    return xs, ys, os_, 2 * l1 + 1, 2 * l3 + 1


def _messages(plan, xe, Ye, we):
    """Per-edge messages [n, outdim] for sender rows xe [n, xdim], Ye, we [n, P, U]."""
    n, U = xe.shape[0], plan.U
    msg = np.zeros((n, plan.outdim))
    for p in range(plan.n_paths):
        xs, ys, os_, da, dc = _blocks(plan, p)
        xa = xe[:, xs].reshape(n, U, da)
        t = np.einsum("abc,eua,eb->euc", plan.cg[p], xa, Ye[:, ys], optimize=True)
        msg[:, os_] += (t * we[:, p, :, None]).reshape(n, U * dc)
    return msg


def _check(plan, src, dst, n_nodes, x, Y):
    src = np.asarray(src, dtype=np.int64)
    dst = np.asarray(dst, dtype=np.int64)
    x = np.asarray(x, dtype=np.float64)
    Y = np.asarray(Y, dtype=np.float64)
    if x.shape != (n_nodes, plan.xdim) or Y.shape != (len(src), plan.ysh):
        raise ValueError("shape mismatch")
    if len(src) and (src.min() < 0 or src.max() >= n_nodes or dst.min() < 0 or dst.max() >= n_nodes):
        raise ValueError("node index out of range")
    return src, dst, x, Y


def tp_conv_fwd(plan, src, dst, n_nodes, x, Y, w):
    """Forward convolution: returns out [n_nodes, outdim] (float64).

    x [N, xdim], Y [E, ysh], w [E, P, U]; edge e goes src[e] -> dst[e].
    """
    src, dst, x, Y = _check(plan, src, dst, n_nodes, x, Y)
    w = np.asarray(w, dtype=np.float64).reshape(len(src), plan.n_paths, plan.U)
    out = np.zeros((n_nodes, plan.outdim))
    for s in range(0, len(src), CHUNK):
        e = slice(s, s + CHUNK)
        np.add.at(out, dst[e], _messages(plan, x[src[e]], Y[e], w[e]))
    return out


def _adjoint_chunk(plan, xe, Ye, we, ge):
    """Adjoint pieces for one chunk: (grad_x rows for senders, grad_Y, grad_w)."""
    n, U = xe.shape[0], plan.U
    gx = np.zeros((n, plan.xdim))
    gY = np.zeros((n, plan.ysh))
    gw = np.zeros((n, plan.n_paths, U))
    for p in range(plan.n_paths):
        xs, ys, os_, da, dc = _blocks(plan, p)
        C = plan.cg[p]
        xa = xe[:, xs].reshape(n, U, da)
        yb = Ye[:, ys]
        gc = ge[:, os_].reshape(n, U, dc)
        wp = we[:, p, :]
        gw[:, p, :] = np.einsum("abc,eua,eb,euc->eu", C, xa, yb, gc, optimize=True)
        gY[:, ys] += np.einsum("abc,eua,euc,eu->eb", C, xa, gc, wp, optimize=True)
        gx[:, xs] += np.einsum("abc,eb,euc,eu->eua", C, yb, gc, wp,
                               optimize=True).reshape(n, U * da)
    return gx, gY, gw


def tp_conv_bwd(plan, src, dst, n_nodes, x, Y, w, g):
    """Gradients of <g, out> with respect to x, Y and w: (grad_x, grad_Y, grad_w)."""
    src, dst, x, Y = _check(plan, src, dst, n_nodes, x, Y)
    w = np.asarray(w, dtype=np.float64).reshape(len(src), plan.n_paths, plan.U)
    g = np.asarray(g, dtype=np.float64)
    grad_x = np.zeros_like(x)
    grad_Y = np.zeros_like(Y)
    grad_w = np.zeros_like(w)
    for s in range(0, len(src), CHUNK):
        e = slice(s, s + CHUNK)
        gx, gY, gw = _adjoint_chunk(plan, x[src[e]], Y[e], w[e], g[dst[e]])
        np.add.at(grad_x, src[e], gx)
        grad_Y[e] = gY
        grad_w[e] = gw
    return grad_x, grad_Y, grad_w


def tp_conv_double_bwd(plan, src, dst, n_nodes, x, Y, w, g, ggx=None, ggY=None, ggw=None):
    """Second-order backward ("Sobek", Abstract: forward, backward and double
    backward).  With F(g, x, Y, w) = <g, out(x, Y, w)> (linear in each
    argument) the first backward returns (gx, gY, gw) = grad F; given
    cotangents (ggx, ggY, ggw) of those (None: zero), the loss
    L = <ggx, gx> + <ggY, gY> + <ggw, gw> equals
        F(g, ggx, Y, w) + F(g, x, ggY, w) + F(g, x, Y, ggw),
    so its gradients are
        dg = out(ggx, Y, w) + out(x, ggY, w) + out(x, Y, ggw)
        dx = gx(ggY, w, g) + gx(Y, ggw, g)     (sender-side adjoint)
        dY = gY(ggx, w, g) + gY(x, ggw, g)     (receiver-side adjoint)
        dw = gw(ggx, Y, g) + gw(x, ggY, g)
    where gx(Y', w', g) is the first backward's grad_x with Y, w replaced, etc.
    Returns (dx, dY, dw, dg)."""
    src, dst, x, Y = _check(plan, src, dst, n_nodes, x, Y)
    w = np.asarray(w, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    z = lambda a, like: np.zeros_like(like) if a is None else np.asarray(a, dtype=np.float64)
    ggx, ggY, ggw = z(ggx, x), z(ggY, Y), z(ggw, w)
    dg = (tp_conv_fwd(plan, src, dst, n_nodes, ggx, Y, w) + tp_conv_fwd(plan, src, dst, n_nodes, x, ggY, w)
          + tp_conv_fwd(plan, src, dst, n_nodes, x, Y, ggw))
    gx_a, gY_a, gw_a = tp_conv_bwd(plan, src, dst, n_nodes, ggx, Y, w, g)      # x -> ggx
    gx_b, gY_b, gw_b = tp_conv_bwd(plan, src, dst, n_nodes, x, ggY, w, g)      # Y -> ggY
    gx_c, gY_c, gw_c = tp_conv_bwd(plan, src, dst, n_nodes, x, Y, ggw, g)      # w -> ggw
    dx = gx_b + gx_c
    dY = gY_a + gY_c
    dw = gw_a + gw_b
    return dx, dY, dw, dg


# ---------------------------------------------------------------------------
# Radial weights (edge-conditioned weights computed from the edge length).
#
# The pages reassociate "radial projection" with the coupling and the
# aggregation so that per-edge weights never exist in memory (Sobek, Abstract
# and AI Summary) but do not define the radial network.  Reading: n_basis
# Bessel functions B_n(r) = sqrt(2/r_c) sin(n pi r / r_c) / r, n = 1..n_basis,
# no envelope; h = SiLU(B W1); w = h W2 with column p*U + u; no biases.
# ---------------------------------------------------------------------------

def bessel_basis(r_len, n_basis, r_cut):
    r = np.asarray(r_len, dtype=np.float64).reshape(-1, 1)
    n = np.arange(1, n_basis + 1, dtype=np.float64).reshape(1, -1)
    return np.sqrt(2.0 / r_cut) * np.sin(n * np.pi * r / r_cut) / r


def bessel_basis_deriv(r_len, n_basis, r_cut):
    """dB_n/dr: sqrt(2/r_c) (k_n cos(k_n r) / r - sin(k_n r) / r^2), k_n = n pi / r_c."""
    r = np.asarray(r_len, dtype=np.float64).reshape(-1, 1)
    k = np.arange(1, n_basis + 1, dtype=np.float64).reshape(1, -1) * np.pi / r_cut
    return np.sqrt(2.0 / r_cut) * (k * np.cos(k * r) / r - np.sin(k * r) / r ** 2)


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def radial_mlp_fwd(r_len, W1, W2, n_basis, r_cut):
    """Edge weights w [E, P*U] and the values the backward needs."""
    B = bessel_basis(r_len, n_basis, r_cut)
    pre = B @ np.asarray(W1, dtype=np.float64)
    h = pre * _sigmoid(pre)
    w = h @ np.asarray(W2, dtype=np.float64)
    return w, (B, pre, h)


def radial_mlp_bwd(grad_w, cache, W2, W1=None):
    """(grad_W1, grad_W2) from grad_w [E, P*U]; with W1 also grad_B [E, n_basis],
    the gradient with respect to the basis values."""
    B, pre, h = cache
    grad_w = np.asarray(grad_w, dtype=np.float64)
    grad_W2 = h.T @ grad_w
    grad_h = grad_w @ np.asarray(W2, dtype=np.float64).T
    s = _sigmoid(pre)
    grad_pre = grad_h * (s * (1.0 + pre * (1.0 - s)))
    grad_W1 = B.T @ grad_pre
    if W1 is None:
        return grad_W1, grad_W2
    return grad_W1, grad_W2, grad_pre @ np.asarray(W1, dtype=np.float64).T


# ---------------------------------------------------------------------------
# Post-aggregation channel mix ("uvw"), one U x U matrix per output irrep:
#   out2[i, k, v, c] = sum_u Wmix[k, u, v] out[i, k, u, c]
# Reading: one matrix per output irrep (not per l) so that 1e and 1o never mix.
# ---------------------------------------------------------------------------

def uvw_mix_fwd(plan, out, Wmix):
    out = np.asarray(out, dtype=np.float64)
    Wmix = np.asarray(Wmix, dtype=np.float64)
    n, U = out.shape[0], plan.U
    out2 = np.zeros_like(out)
    for k, (l, _) in enumerate(plan.out_irreps):
        s = slice(plan.out_offsets[k], plan.out_offsets[k] + U * (2 * l + 1))
        blk = out[:, s].reshape(n, U, 2 * l + 1)
        out2[:, s] = np.einsum("uv,nuc->nvc", Wmix[k], blk).reshape(n, -1)
    return out2


def uvw_mix_bwd(plan, out, Wmix, g2):
    """(grad_out, grad_Wmix) of <g2, uvw_mix_fwd(out)>."""
    out = np.asarray(out, dtype=np.float64)
    g2 = np.asarray(g2, dtype=np.float64)
    Wmix = np.asarray(Wmix, dtype=np.float64)
    n, U = out.shape[0], plan.U
    grad_out = np.zeros_like(out)
    grad_W = np.zeros_like(Wmix)
    for k, (l, _) in enumerate(plan.out_irreps):
        s = slice(plan.out_offsets[k], plan.out_offsets[k] + U * (2 * l + 1))
        o = out[:, s].reshape(n, U, 2 * l + 1)
        g = g2[:, s].reshape(n, U, 2 * l + 1)
        grad_out[:, s] = np.einsum("uv,nvc->nuc", Wmix[k], g).reshape(n, -1)
        grad_W[k] = np.einsum("nuc,nvc->uv", o, g)
    return grad_out, grad_W


# ---------------------------------------------------------------------------
# Radial-weight convolution: w comes from the radial MLP of the edge length,
# followed by the optional uvw mix.  Edge weights are built per chunk only.
# ---------------------------------------------------------------------------

def tp_conv_radial_fwd(plan, src, dst, n_nodes, x, Y, r_len, W1, W2, Wmix,
                       n_basis, r_cut, return_pre_mix=False):
    src, dst, x, Y = _check(plan, src, dst, n_nodes, x, Y)
    r_len = np.asarray(r_len, dtype=np.float64)
    out = np.zeros((n_nodes, plan.outdim))
    for s in range(0, len(src), CHUNK):
        e = slice(s, s + CHUNK)
        w, _ = radial_mlp_fwd(r_len[e], W1, W2, n_basis, r_cut)
        w = w.reshape(-1, plan.n_paths, plan.U)
        np.add.at(out, dst[e], _messages(plan, x[src[e]], Y[e], w))
    out2 = uvw_mix_fwd(plan, out, Wmix) if Wmix is not None else out
    return (out2, out) if return_pre_mix else out2


def tp_conv_radial_bwd(plan, src, dst, n_nodes, x, Y, r_len, W1, W2, Wmix, g2,
                       n_basis, r_cut, with_grad_rlen=False):
    """(grad_x, grad_Y, grad_W1, grad_W2, grad_Wmix); grad_Wmix is None without a mix.
    with_grad_rlen: a sixth entry, the gradient with respect to the edge lengths
    (through the radial basis), grad_rlen[e] = sum_n grad_B[e, n] dB_n/dr."""
    src, dst, x, Y = _check(plan, src, dst, n_nodes, x, Y)
    r_len = np.asarray(r_len, dtype=np.float64)
    g2 = np.asarray(g2, dtype=np.float64)
    grad_Wmix = None
    if Wmix is not None:
        out = tp_conv_radial_fwd(plan, src, dst, n_nodes, x, Y, r_len, W1, W2,
                                 None, n_basis, r_cut)
        g, grad_Wmix = uvw_mix_bwd(plan, out, Wmix, g2)
    else:
        g = g2
    grad_x = np.zeros_like(x)
    grad_Y = np.zeros_like(Y)
    grad_W1 = np.zeros_like(np.asarray(W1, dtype=np.float64))
    grad_W2 = np.zeros_like(np.asarray(W2, dtype=np.float64))
    grad_rlen = np.zeros(len(src))
    for s in range(0, len(src), CHUNK):
        e = slice(s, s + CHUNK)
        w, cache = radial_mlp_fwd(r_len[e], W1, W2, n_basis, r_cut)
        w = w.reshape(-1, plan.n_paths, plan.U)
        gx, gY, gw = _adjoint_chunk(plan, x[src[e]], Y[e], w, g[dst[e]])
        np.add.at(grad_x, src[e], gx)
        grad_Y[e] = gY
        a, b, gB = radial_mlp_bwd(gw.reshape(gw.shape[0], -1), cache, W2, W1)
        grad_W1 += a
        grad_W2 += b
        grad_rlen[e] = np.sum(gB * bessel_basis_deriv(r_len[e], n_basis, r_cut), axis=1)
    if with_grad_rlen:
        return grad_x, grad_Y, grad_W1, grad_W2, grad_Wmix, grad_rlen
    return grad_x, grad_Y, grad_W1, grad_W2, grad_Wmix


# ---------------------------------------------------------------------------
# Second-order backward of the radial-weight convolution ("Sobek", Abstract:
# forward, backward and double backward, with the radial projection streamed
# so that edge weights never exist in memory).
#
# Reading: the cotangents are those a loss on forces produces -- on the first
# backward's node gradient grad_x, its harmonic gradient grad_Y and its length
# gradient grad_rlen (the edge-vector gradient is built from the last two).
# Cotangents of the parameter gradients (grad_W1, grad_W2, grad_Wmix) are not
# taken: training differentiates a loss on forces, never one on parameter
# gradients.
# ---------------------------------------------------------------------------

def bessel_basis_deriv2(r_len, n_basis, r_cut):
    """d^2 B_n / dr^2 = sqrt(2/r_c) (-k^2 sin(kr)/r - 2k cos(kr)/r^2 + 2 sin(kr)/r^3)."""
    r = np.asarray(r_len, dtype=np.float64).reshape(-1, 1)
    k = np.arange(1, n_basis + 1, dtype=np.float64).reshape(1, -1) * np.pi / r_cut
    s, c = np.sin(k * r), np.cos(k * r)
    return np.sqrt(2.0 / r_cut) * (-k * k * s / r - 2.0 * k * c / r ** 2 + 2.0 * s / r ** 3)


def silu_derivs(z):
    """(SiLU(z), SiLU'(z), SiLU''(z)) with SiLU(z) = z sigma(z):
    SiLU' = sigma (1 + z (1 - sigma)), SiLU'' = sigma (1 - sigma) (2 + z (1 - 2 sigma))."""
    z = np.asarray(z, dtype=np.float64)
    s = _sigmoid(z)
    return z * s, s * (1.0 + z * (1.0 - s)), s * (1.0 - s) * (2.0 + z * (1.0 - 2.0 * s))


def tp_conv_radial_double_bwd(plan, src, dst, n_nodes, x, Y, r_len, W1, W2, Wmix, g2,
                              n_basis, r_cut, ggx=None, ggY=None, ggr=None):
    """Gradients of L = <ggx, grad_x> + <ggY, grad_Y> + <ggr, grad_rlen>, the
    first backward's outputs (``tp_conv_radial_bwd`` with ``with_grad_rlen``),
    with respect to x, Y, r_len, W1, W2, Wmix and the upstream gradient g2.
    Missing cotangents (None) are zero.

    With g = mix^T(g2) the unmixed upstream gradient and F(g, x, Y, w) =
    <g, out(x, Y, w)> (linear in each argument), grad_rlen[e] =
    <dw_e/dr_e, grad_w_e>, so
        L = F(g, ggx, Y, w) + F(g, x, ggY, w) + F(g, x, Y, v),
        v[e] = ggr[e] dw_e/dr_e     (the tangent of the weights along ggr).
    Hence, with out_dot = out(ggx, Y, w) + out(x, ggY, w) + out(x, Y, v):
        d_g2 = mix(out_dot), d_Wmix = grad_Wmix of <g2, mix(out_dot)>,
        dx = gx(ggY, w, g) + gx(Y, v, g),  dY = gY(ggx, w, g) + gY(x, v, g),
    and the weights' cotangent dw = gw(ggx, Y, g) + gw(x, ggY, g) and the
    tangent's cotangent dv = gw(x, Y, g) flow back through the network
    pre = B W1, h = SiLU(pre), w = h W2, a = B' W1, t = SiLU'(pre) a,
    v = ggr t W2 by the chain rule, which is where SiLU'' and B'' enter.
    Returns (dx, dY, d_rlen, dW1, dW2, dWmix, d_g2); dWmix is None without a
    mix."""
    src, dst, x, Y = _check(plan, src, dst, n_nodes, x, Y)
    E = len(src)
    r_len = np.asarray(r_len, dtype=np.float64)
    W1 = np.asarray(W1, dtype=np.float64)
    W2 = np.asarray(W2, dtype=np.float64)
    g2 = np.asarray(g2, dtype=np.float64)
    z = lambda a, like: np.zeros_like(like) if a is None else np.asarray(a, dtype=np.float64)
    ggx, ggY, ggr = z(ggx, x), z(ggY, Y), z(ggr, r_len)
    if Wmix is not None:
        g, _ = uvw_mix_bwd(plan, np.zeros_like(g2), Wmix, g2)
    else:
        g = g2
    # the network, its derivative in r and the weight tangent
    B = bessel_basis(r_len, n_basis, r_cut)
    dB = bessel_basis_deriv(r_len, n_basis, r_cut)
    d2B = bessel_basis_deriv2(r_len, n_basis, r_cut)
    pre = B @ W1
    h, s1, s2 = silu_derivs(pre)
    a = dB @ W1                                   # d pre / dr
    t = s1 * a                                    # d h / dr
    w = (h @ W2).reshape(E, plan.n_paths, plan.U)
    v = ((ggr[:, None] * t) @ W2).reshape(E, plan.n_paths, plan.U)
    args = (plan, src, dst, n_nodes)
    out_dot = (tp_conv_fwd(*args, ggx, Y, w) + tp_conv_fwd(*args, x, ggY, w)
               + tp_conv_fwd(*args, x, Y, v))
    if Wmix is not None:
        d_g2 = uvw_mix_fwd(plan, out_dot, Wmix)
        _, dWmix = uvw_mix_bwd(plan, out_dot, Wmix, g2)
    else:
        d_g2, dWmix = out_dot, None
    _, gY_a, gw_a = tp_conv_bwd(*args, ggx, Y, w, g)      # x -> ggx
    gx_b, _, gw_b = tp_conv_bwd(*args, x, ggY, w, g)      # Y -> ggY
    gx_c, gY_c, gw_c = tp_conv_bwd(*args, x, Y, v, g)     # w -> v
    dx = gx_b + gx_c
    dY = gY_a + gY_c
    dw = (gw_a + gw_b).reshape(E, -1)
    dv = gw_c.reshape(E, -1)
    # back through the network
    dW2 = h.T @ dw + (ggr[:, None] * t).T @ dv
    dh = dw @ W2.T
    dt = ggr[:, None] * (dv @ W2.T)
    dpre = s1 * dh + s2 * a * dt
    da = s1 * dt
    dW1 = B.T @ dpre + dB.T @ da
    d_rlen = np.sum(dB * (dpre @ W1.T), axis=1) + np.sum(d2B * (da @ W1.T), axis=1)
    return dx, dY, d_rlen, dW1, dW2, dWmix, d_g2
