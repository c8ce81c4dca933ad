// Gaunt (spherical-grid) tensor-product convolution: a different operator from
// the Clebsch-Gordan convolution, cheaper and less expressive ("The Price of
// Freedom: Exploring Expressivity and Runtime Tradeoffs in Equivariant Tensor
// Products", Abstract: the Gaunt product evaluated directly on a spherical
// grid).
//
// Per channel u the sender's features are the signal
//   f_{j,u}(s) = sum_{l,m} x[j, l, u, m] Y_lm(s),
// the edge carries the filter
//   g_{e,u}(s) = sum_{l2} w[e][l2][u] Z_{e,l2}(s),   Z_{e,l2}(s) = sum_m Y[e][l2,m] Y_{l2 m}(s),
// and the receiver gets the harmonic coefficients of sum_e f g:
//   out[i, l3, u, m3] = (1/4pi) int Y_{l3 m3}(s) H_{i,u}(s) dOmega,
//   H_{i,u}(s) = sum_{e = (j -> i)} f_{j,u}(s) g_{e,u}(s).
// All three stages are evaluated on one product grid, 4 Gauss-Legendre nodes
// in cos(theta) times 8 equispaced azimuths (32 points, exact for total degree
// 7 >= 2 + 2 + 2), so the result equals the coefficient sum with the Gaunt
// coefficients up to rounding.  The projection is linear, so it moves out of
// the edge sum and runs once per receiver.
//
// Per edge the two signals on the grid are dense contractions, run on the
// matrix cores (v_mfma_f32_32x32x2f32, 32 channels x 32 points per wave):
//   f[u][q] = sum_a x[j][u][a] Yq[a][q]        (K = 9 harmonics, padded to 10)
//   g[u][q] = sum_l2 w[e][l2][u] Z[l2][q]      (K = lmax_sh + 1, padded to 4)
// and H += f * g elementwise in the accumulator layout (both products share
// it).  The sender's row x_j (9 numbers per channel) is gathered directly; it
// is small enough to stay in every XCD's L2, unlike x expanded onto the grid
// (3.6 times larger), which would be gathered from beyond the L2.
//
// Workgroup = one receiver; U <= 32: two waves split the receiver's edges;
// U = 64 / 128: two / four 32-channel tiles, the two / one waves of a tile
// split the edges.  The waves meet in LDS, the projection onto the output harmonics
// runs on the vector units and each output row is written once: no per-edge
// message, no atomics, a fixed summation order.
#include <cmath>

#include "internal.hpp"

namespace tpc {
namespace {

constexpr int kQ = 32;        // grid points
constexpr int kNT = 4;        // Gauss-Legendre nodes in cos(theta)
constexpr int kNP = 8;        // azimuths
constexpr int kHS = 36;       // LDS row stride of the grid accumulator and projector
constexpr int kPipe = 2;      // edges per pipelined batch of one wave
constexpr int kChunk = 256;   // edges whose sender index and Y row are staged in LDS at a time

typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

struct GauntLayout {
  int n_in;         // input irreps (distinct degrees <= 2)
  int deg[3];
  int off[3];       // column of each input block in a node row
  int xdim, ysh, lout, outdim;
};

// ---- the grid, built at compile time ------------------------------------------
// 4-point Gauss-Legendre rule in t = cos(theta) (closed form: nodes
// +-sqrt(3/7 -+ (2/7) sqrt(6/5)), weights (18 +- sqrt 30) / 36) times the 8
// azimuths 2 pi b / 8, whose cosines and sines are 0, +-1 and +-sqrt(1/2).
constexpr double csqrt(double v) {
  double r = v > 1.0 ? v : 1.0;
  for (int it = 0; it < 60; ++it) r = 0.5 * (r + v / r);
  return r;
}

struct GridTab {
  float y[10][kQ];   // Y_c(s_q), c = l^2 + m (l <= 2); row 9 is the K padding (zero)
  float p[9][kQ];    // (1/4pi) x quadrature weight x Y_c(s_q)
};

constexpr GridTab make_grid() {
  GridTab g{};
  const double a = 2.0 / 7.0 * csqrt(6.0 / 5.0), s30 = csqrt(30.0);
  const double t[kNT] = {-csqrt(3.0 / 7.0 + a), -csqrt(3.0 / 7.0 - a), csqrt(3.0 / 7.0 - a),
                         csqrt(3.0 / 7.0 + a)};
  const double wt[kNT] = {(18.0 - s30) / 36.0, (18.0 + s30) / 36.0, (18.0 + s30) / 36.0,
                          (18.0 - s30) / 36.0};
  const double r2 = csqrt(0.5);
  const double cb[kNP] = {1.0, r2, 0.0, -r2, -1.0, -r2, 0.0, r2};
  const double sb[kNP] = {0.0, r2, 1.0, r2, 0.0, -r2, -1.0, -r2};
  const double s3 = csqrt(3.0), s15 = csqrt(15.0), s5 = csqrt(5.0);
  for (int ia = 0; ia < kNT; ++ia)
    for (int ib = 0; ib < kNP; ++ib) {
      const int q = ia * kNP + ib;
      const double st = csqrt(1.0 - t[ia] * t[ia]);
      const double x = st * cb[ib], y = st * sb[ib], z = t[ia];
      const double v[9] = {1.0,           s3 * y,        s3 * z,
                           s3 * x,        s15 * x * y,   s15 * y * z,
                           0.5 * s5 * (3.0 * z * z - 1.0), s15 * x * z,
                           0.5 * s15 * (x * x - y * y)};
      const double wq = wt[ia] / (2.0 * kNP);   // (1/4pi) * Gauss weight * (2pi / azimuths)
      for (int c = 0; c < 9; ++c) {
        g.y[c][q] = (float)v[c];
        g.p[c][q] = (float)(wq * v[c]);
      }
      g.y[9][q] = 0.f;
    }
  return g;
}

__constant__ GridTab c_grid = make_grid();

__device__ __forceinline__ v16f mfma32(float a, float b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// v_mfma_f32_32x32x2f32 operand and result layouts (lane l, k = l / 32):
//   A[i][k] from lane i + 32 k, B[k][j] from lane j + 32 k,
//   D[i][j] in lane j + 32 ((i / 4) % 2), register (i % 4) + 4 (i / 8).
template <int U, int NL2, int WPT>
__global__ void __launch_bounds__(64 * (U >= 32 ? U / 32 : 1) * WPT)
    k_gaunt_conv(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col,
                 const float* __restrict__ x, const float* __restrict__ Y, const float* __restrict__ w,
                 float* __restrict__ out, GauntLayout L,
                 const int32_t* __restrict__ order) {
  constexpr int NUT = U >= 32 ? U / 32 : 1;       // 32-channel tiles
  constexpr int NW = NUT * WPT;                   // waves (WPT per tile)
  constexpr int NTH = 64 * NW;
  constexpr int WD = NL2 * U;                     // weights per edge
  __shared__ __align__(16) float ps[9][kHS];
  __shared__ __align__(16) float hs[NW][32][kHS];
  __shared__ int cs[kChunk];
  __shared__ float ysm[kChunk * 9];
  // node of this workgroup in the launch order (largest degree first), or node order
  const int i = order ? min(max(order[blockIdx.x], 0), (int)gridDim.x - 1) : (int)blockIdx.x, t = threadIdx.x;
  const int beg = row_ptr[i], end = row_ptr[i + 1];
  const int wave = __builtin_amdgcn_readfirstlane(t / 64), lane = t % 64;
  const int ut = wave / WPT, sub = wave % WPT;
  const int n = lane % 32, hk = lane / 32;
  float yv[9];
#pragma unroll
  for (int c = 0; c < 9; ++c) yv[c] = c_grid.y[c][n];      // harmonics at this lane's point
  for (int k = t; k < 9 * kQ; k += NTH) ps[k / kQ][k % kQ] = c_grid.p[k / kQ][k % kQ];
  // f = A_x B_Y with K index a = 2 ks + hk: B[a][q] = Yq[a][q], zero for the
  // padding a = 9 and for degrees the input lacks (their A entries are then
  // any finite in-row value); A[u][a] = x[j][block of degree l(a)][u][m(a)].
  // Rows u >= U (U = 16) read channel U - 1 and are never stored.
  const int u = 32 * ut + n, uc = u < U ? u : U - 1;
  float bf[5];
  int xo[5];
#pragma unroll
  for (int ks = 0; ks < 5; ++ks) {
    const int a = 2 * ks + hk;
    const int l = a == 0 ? 0 : (a < 4 ? 1 : 2), m = a - l * l;
    int o = -1;
    for (int b = 0; b < L.n_in; ++b)
      if (L.deg[b] == l && a < 9) o = L.off[b] + uc * (2 * l + 1) + m;
    bf[ks] = o >= 0 ? c_grid.y[a][n] : 0.f;
    xo[ks] = o >= 0 ? o : 0;
  }
  // g = A_w B_Z with K index l2 = 2 ks + hk (ks = 0, 1): A[u][l2] = w[e][l2][u],
  // B[l2][q] = Z[l2][q], zero for l2 >= NL2 (then A reads a finite in-row value)
  int wo[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) wo[ks] = (2 * ks + hk < NL2 ? (2 * ks + hk) * U : 0) + uc;

  v16f h, zero;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    h[r] = 0.f;
    zero[r] = 0.f;
  }
  // The receiver's sender indices and Y rows are staged in LDS (chunks of
  // kChunk edges); each wave walks its edges (wave-uniform) a pair at a time
  // with two pair buffers, so one pair's gathers are in flight while the
  // other's products run.  Every fetch is issued (the index is clamped to the
  // chunk) so the number of loads in flight is the same on every path.
  struct Ops {
    float x[5], w[2];
  };
  auto fetch = [&](int c0, int k, Ops& o) {
    const float* xj = x + (size_t)cs[k] * L.xdim;
    const float* we = w + (size_t)(c0 + k) * WD;
#pragma unroll
    for (int ks = 0; ks < 5; ++ks) o.x[ks] = xj[xo[ks]];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) o.w[ks] = __builtin_nontemporal_load(we + wo[ks]);
  };
  // Z[l2][q] = sum_m Y[e][l2, m] Yq[l2, m][q] at this lane's point, as the
  // B operand of the filter product (K index l2 = 2 ks + hk)
  auto zval = [&](int k, float valid, float& zb0, float& zb1) {
    const float* yk = ysm + k * L.ysh;
    float z[3] = {0.f, 0.f, 0.f};
#pragma unroll
    for (int l2 = 0; l2 < NL2; ++l2)
#pragma unroll
      for (int m = 0; m < 2 * l2 + 1; ++m) z[l2] = fmaf(yk[l2 * l2 + m], yv[l2 * l2 + m], z[l2]);
    zb0 = (hk ? z[1] : z[0]) * valid;
    zb1 = hk ? 0.f : z[2] * valid;
  };
  // two edges' products, interleaved so the two dependent chains overlap
  auto product2 = [&](const Ops& o0, int k0, float v0, const Ops& o1, int k1, float v1) {
    float za0, za1, zc0, zc1;
    zval(k0, v0, za0, za1);
    zval(k1, v1, zc0, zc1);
    v16f f0 = mfma32(o0.x[0], bf[0], zero);
    v16f f1 = mfma32(o1.x[0], bf[0], zero);
#pragma unroll
    for (int ks = 1; ks < 5; ++ks) {
      f0 = mfma32(o0.x[ks], bf[ks], f0);
      f1 = mfma32(o1.x[ks], bf[ks], f1);
    }
    v16f g0 = mfma32(o0.w[0], za0, zero);
    v16f g1 = mfma32(o1.w[0], zc0, zero);
    g0 = mfma32(o0.w[1], za1, g0);
    g1 = mfma32(o1.w[1], zc1, g1);
#pragma unroll
    for (int r = 0; r < 16; ++r) h[r] = fmaf(f0[r], g0[r], fmaf(f1[r], g1[r], h[r]));
  };
  for (int c0 = beg; c0 < end; c0 += kChunk) {
    const int cn = end - c0 < kChunk ? end - c0 : kChunk;
    __syncthreads();   // previous chunk consumed
    for (int k = t; k < cn; k += NTH) cs[k] = col[c0 + k];
    for (int k = t; k < cn * L.ysh; k += NTH) ysm[k] = Y[(size_t)c0 * L.ysh + k];
    __syncthreads();
    // pairs of edges per wave, software-pipelined: the gathers of the next
    // pair are issued before the products of this one, which then wait for
    // their own loads only (loads complete in order); 29 against 31 us for
    // batches of eight loaded and then computed.  Slots past the chunk's end
    // re-read its last edge and are multiplied by zero (every load is issued,
    // so the counts in flight are the same on every path).
    constexpr int B = kPipe;
    auto fetch_batch = [&](int k0, Ops (&o)[B]) {
#pragma unroll
      for (int r = 0; r < B; ++r) fetch(c0, k0 + r * WPT < cn ? k0 + r * WPT : cn - 1, o[r]);
    };
    auto compute_batch = [&](int k0, const Ops (&o)[B]) {
#pragma unroll
      for (int r = 0; r < B; r += 2) {
        const bool ok0 = k0 + r * WPT < cn, ok1 = k0 + (r + 1) * WPT < cn;
        product2(o[r], ok0 ? k0 + r * WPT : cn - 1, ok0 ? 1.f : 0.f, o[r + 1],
                 ok1 ? k0 + (r + 1) * WPT : cn - 1, ok1 ? 1.f : 0.f);
      }
    };
    if (sub < cn) {
      Ops oa[B], ob[B];
      fetch_batch(sub, oa);
      for (int k0 = sub; k0 < cn; k0 += 2 * B * WPT) {
        fetch_batch(k0 + B * WPT, ob);
        __builtin_amdgcn_sched_barrier(0);
        compute_batch(k0, oa);
        if (k0 + B * WPT >= cn) break;
        fetch_batch(k0 + 2 * B * WPT, oa);
        __builtin_amdgcn_sched_barrier(0);
        compute_batch(k0 + B * WPT, ob);
      }
    }
  }
  // D[row][col = q]: row = 8 (r / 4) + 4 hk + r % 4 (channel within the tile)
#pragma unroll
  for (int r = 0; r < 16; ++r) hs[wave][8 * (r / 4) + 4 * hk + r % 4][n] = h[r];
  __syncthreads();
  if (WPT > 1) {   // the waves of a tile add up, once, into the tile's first copy
    for (int k = t; k < NUT * 32 * 32; k += NTH) {
      const int tw = (k / 1024) * WPT, row = (k / 32) % 32, q = k % 32;
      float a = hs[tw][row][q];
#pragma unroll
      for (int s2 = 1; s2 < WPT; ++s2) a += hs[tw + s2][row][q];
      hs[tw][row][q] = a;
    }
    __syncthreads();
  }
  // projection onto the output harmonics; block l3 starts at column U l3^2,
  // channel uu's components at uu (2 l3 + 1)
  for (int o = t; o < L.outdim; o += NTH) {
    const int l3 = o < U ? 0 : (o < 4 * U ? 1 : 2);
    const int d = 2 * l3 + 1, r = o - U * l3 * l3;
    const int uu = r / d, c = l3 * l3 + (r - uu * d);
    const float4* hr = reinterpret_cast<const float4*>(hs[(uu / 32) * WPT][uu % 32]);
    const float4* pr = reinterpret_cast<const float4*>(ps[c]);
    float a = 0.f;
#pragma unroll
    for (int k = 0; k < kQ / 4; ++k) {
      const float4 hv = hr[k], pv = pr[k];
      a = fmaf(hv.x, pv.x, a);
      a = fmaf(hv.y, pv.y, a);
      a = fmaf(hv.z, pv.z, a);
      a = fmaf(hv.w, pv.w, a);
    }
    out[(size_t)i * L.outdim + o] = a;
  }
}

// ---- backward --------------------------------------------------------------
// With gH_i[u][q] = sum_c P[c][q] gout_i[u][c] (the adjoint of the projection)
// and the forward's signals f (sender) and g (filter) on the grid:
//   grad_x[j][u][a]  = sum_q Yq[a][q] sum_{e = (j -> i)} gH_i[u][q] g_e[u][q]      (sender pass)
//   grad_w[e][l2][u] = sum_q gH_i[u][q] f_j[u][q] Z_e[l2][q]                      (receiver pass)
//   grad_Y[e][l2,m]  = sum_q Yq[l2m][q] sum_u gH_i[u][q] f_j[u][q] w_e[l2][u]     (receiver pass)
// gH is one more 32x32x2 product per 32-channel tile (K = output harmonics).

// A operand of a product over an output row (K index c = 2 ks + hk, padded to
// 10): this lane's column offsets and the matching B values of a table
__device__ __forceinline__ void out_operand(const GauntLayout& L, int U, int uc, int hk, int n,
                                            const float (&tab)[9][kQ], int (&oo)[5], float (&bt)[5]) {
  const int nc = (L.lout + 1) * (L.lout + 1);
#pragma unroll
  for (int ks = 0; ks < 5; ++ks) {
    const int c = 2 * ks + hk;
    const int l3 = c == 0 ? 0 : (c < 4 ? 1 : 2), m = c - l3 * l3;
    const bool ok = c < nc;
    oo[ks] = ok ? U * l3 * l3 + uc * (2 * l3 + 1) + m : 0;
    bt[ks] = ok ? tab[c < 9 ? c : 8][n] : 0.f;
  }
}

// Receiver pass: grad_w and grad_Y (either may be skipped).  One workgroup per
// receiver; its four waves split the edges and every wave covers all channel
// tiles.  Per edge and tile: f (five products), gg = gH f (elementwise); the
// sum over channels for grad_Y is in-lane (the lane's 16 channels) plus one
// cross-half exchange, then a butterfly over the 32 points; the sum over
// points for grad_w goes through a per-wave LDS transpose of gg.
template <int U, int NL2, int NW>
__global__ void __launch_bounds__(64 * NW)
    k_gaunt_bwd_recv(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col,
                     const float* __restrict__ x, const float* __restrict__ Y, const float* __restrict__ w,
                     const float* __restrict__ gout, float* __restrict__ grad_Y, float* __restrict__ grad_w,
                     GauntLayout L, const int32_t* __restrict__ order) {
  constexpr int NUT = U >= 32 ? U / 32 : 1;
  constexpr int WD = NL2 * U;
  constexpr int YS = NL2 * NL2;
  constexpr int CR = WD <= 128 ? 32 : (WD <= 256 ? 16 : 8);   // edges staged per chunk
  __shared__ int cs[CR];
  __shared__ float ysm[CR * 9];
  __shared__ __align__(16) float wsm[CR * WD];
  __shared__ __align__(16) float tr[NW][32][kHS];     // per-wave transpose of gg
  __shared__ __align__(16) float zt[NW][3][kQ];       // per-wave Z at the 32 points
  __shared__ __align__(16) float yr[NW][9][kHS];      // per-wave grad_Y terms at the 32 points
  // node of this workgroup in the launch order (largest degree first), or node order
  const int i = order ? min(max(order[blockIdx.x], 0), (int)gridDim.x - 1) : (int)blockIdx.x, t = threadIdx.x;
  const int beg = row_ptr[i], end = row_ptr[i + 1];
  const int wave = __builtin_amdgcn_readfirstlane(t / 64), lane = t % 64;
  const int n = lane % 32, hk = lane / 32;
  float yv[9];
#pragma unroll
  for (int c = 0; c < 9; ++c) yv[c] = c_grid.y[c][n];
  v16f zero;
#pragma unroll
  for (int r = 0; r < 16; ++r) zero[r] = 0.f;
  // per tile: gH (this receiver's output gradient on the grid) and the
  // operands of f
  v16f gH[NUT];
  int xo[NUT][5];
  float bf[5];
#pragma unroll
  for (int ut = 0; ut < NUT; ++ut) {
    const int u = 32 * ut + n, uc = u < U ? u : U - 1;
    int oo[5];
    float bp[5];
    out_operand(L, U, uc, hk, n, c_grid.p, oo, bp);
    gH[ut] = zero;
#pragma unroll
    for (int ks = 0; ks < 5; ++ks) gH[ut] = mfma32(gout[(size_t)i * L.outdim + oo[ks]], bp[ks], gH[ut]);
#pragma unroll
    for (int ks = 0; ks < 5; ++ks) {
      const int a = 2 * ks + hk;
      const int l = a == 0 ? 0 : (a < 4 ? 1 : 2), m = a - l * l;
      int o = -1;
      for (int b = 0; b < L.n_in; ++b)
        if (L.deg[b] == l && a < 9) o = L.off[b] + uc * (2 * l + 1) + m;
      if (ut == 0) bf[ks] = o >= 0 ? c_grid.y[a][n] : 0.f;
      xo[ut][ks] = o >= 0 ? o : 0;
    }
  }
  // one edge (k in the chunk, its sender row gathered in xa) for every tile
  auto edge = [&](int c0, int k, const float (&xa)[NUT][5]) {
    const size_t e = (size_t)(c0 + k);
    float z[3] = {0.f, 0.f, 0.f};
#pragma unroll
    for (int l2 = 0; l2 < NL2; ++l2)
#pragma unroll
      for (int m = 0; m < 2 * l2 + 1; ++m) z[l2] = fmaf(ysm[k * L.ysh + l2 * l2 + m], yv[l2 * l2 + m], z[l2]);
    if (grad_w && hk == 0) {
#pragma unroll
      for (int l2 = 0; l2 < NL2; ++l2) zt[wave][l2][n] = z[l2];
    }
    float gz[3] = {0.f, 0.f, 0.f};
#pragma unroll
    for (int ut = 0; ut < NUT; ++ut) {
      v16f f = mfma32(xa[ut][0], bf[0], zero);
#pragma unroll
      for (int ks = 1; ks < 5; ++ks) f = mfma32(xa[ut][ks], bf[ks], f);
      v16f gg;
#pragma unroll
      for (int r = 0; r < 16; ++r) gg[r] = gH[ut][r] * f[r];
      // rows of register r: channel 32 ut + 8 (r / 4) + 4 hk + r % 4
      if (grad_Y) {
#pragma unroll
        for (int l2 = 0; l2 < NL2; ++l2)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int u0 = 32 * ut + 8 * q4 + 4 * hk;
            if (u0 < U) {
              const float4 w4 = *reinterpret_cast<const float4*>(&wsm[k * WD + l2 * U + u0]);
              gz[l2] = fmaf(gg[4 * q4], w4.x, gz[l2]);
              gz[l2] = fmaf(gg[4 * q4 + 1], w4.y, gz[l2]);
              gz[l2] = fmaf(gg[4 * q4 + 2], w4.z, gz[l2]);
              gz[l2] = fmaf(gg[4 * q4 + 3], w4.w, gz[l2]);
            }
          }
      }
      if (grad_w) {
        // transpose gg through LDS: lane (point n, half hk) writes its 16
        // channels; lane (channel n, half hk) then reads points 16 hk .. +15
#pragma unroll
        for (int r = 0; r < 16; ++r) tr[wave][8 * (r / 4) + 4 * hk + r % 4][n] = gg[r];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float gw[3] = {0.f, 0.f, 0.f};
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const float4 v = reinterpret_cast<const float4*>(&tr[wave][n][16 * hk])[s4];
#pragma unroll
          for (int l2 = 0; l2 < NL2; ++l2) {
            const float4 zz = reinterpret_cast<const float4*>(&zt[wave][l2][16 * hk])[s4];
            gw[l2] = fmaf(v.x, zz.x, fmaf(v.y, zz.y, fmaf(v.z, zz.z, fmaf(v.w, zz.w, gw[l2]))));
          }
        }
#pragma unroll
        for (int l2 = 0; l2 < NL2; ++l2) gw[l2] += __shfl_xor(gw[l2], 32, 64);
        if (hk == 0 && 32 * ut + n < U) {
#pragma unroll
          for (int l2 = 0; l2 < NL2; ++l2) grad_w[e * WD + l2 * U + 32 * ut + n] = gw[l2];
        }
        __builtin_amdgcn_wave_barrier();
      }
    }
    if (grad_Y) {
      // channels of the other half; then the terms Yq[c][q] gZ[l2(c)][q] go
      // through LDS and lane c < ysh adds its row over the 32 points
#pragma unroll
      for (int l2 = 0; l2 < NL2; ++l2) gz[l2] += __shfl_xor(gz[l2], 32, 64);
      if (hk == 0) {
#pragma unroll
        for (int c = 0; c < YS; ++c) yr[wave][c][n] = yv[c] * gz[c == 0 ? 0 : (c < 4 ? 1 : 2)];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int c = n < YS ? n : 0;
      float acc = 0.f;
#pragma unroll
      for (int s4 = 0; s4 < kQ / 4; ++s4) {
        const float4 v = reinterpret_cast<const float4*>(yr[wave][c])[s4];
        acc += (v.x + v.y) + (v.z + v.w);
      }
      if (hk == 0 && n < YS) grad_Y[e * L.ysh + n] = acc;
      __builtin_amdgcn_wave_barrier();
    }
  };
  for (int c0 = beg; c0 < end; c0 += CR) {
    const int cn = end - c0 < CR ? end - c0 : CR;
    __syncthreads();   // previous chunk consumed
    for (int k = t; k < cn; k += 64 * NW) cs[k] = col[c0 + k];
    for (int k = t; k < cn * L.ysh; k += 64 * NW) ysm[k] = Y[(size_t)c0 * L.ysh + k];
    {
      const float4* src = reinterpret_cast<const float4*>(w + (size_t)c0 * WD);
      for (int k = t; k < cn * WD / 4; k += 64 * NW) reinterpret_cast<float4*>(wsm)[k] = src[k];
    }
    __syncthreads();
    // batches of PB edges per wave, software-pipelined: the sender rows of
    // the next batch are gathered while this batch's products run (slots past
    // the chunk re-read its last edge, unused); one edge per batch measured
    // best (46.6 against 47.3 us for batches of four gathered, then used)
    constexpr int PB = 1;
    auto gather = [&](int k0, float (&xa)[PB][NUT][5]) {
#pragma unroll
      for (int r = 0; r < PB; ++r) {
        const int k = k0 + NW * r < cn ? k0 + NW * r : cn - 1;
        const float* xj = x + (size_t)cs[k] * L.xdim;
#pragma unroll
        for (int ut = 0; ut < NUT; ++ut)
#pragma unroll
          for (int ks = 0; ks < 5; ++ks) xa[r][ut][ks] = xj[xo[ut][ks]];
      }
    };
    auto run = [&](int k0, const float (&xa)[PB][NUT][5]) {
#pragma unroll
      for (int r = 0; r < PB; ++r)
        if (k0 + NW * r < cn) edge(c0, k0 + NW * r, xa[r]);
    };
    if (wave < cn) {
      float xa[PB][NUT][5], xb[PB][NUT][5];
      gather(wave, xa);
      for (int k0 = wave; k0 < cn; k0 += 2 * NW * PB) {
        gather(k0 + NW * PB, xb);
        __builtin_amdgcn_sched_barrier(0);
        run(k0, xa);
        if (k0 + NW * PB >= cn) break;
        gather(k0 + 2 * NW * PB, xa);
        __builtin_amdgcn_sched_barrier(0);
        run(k0 + NW * PB, xb);
      }
    }
  }
}

// Sender pass: grad_x.  The mirror of the forward: one workgroup per sender,
// edges from the sender grouping (receiver-order position t_perm, receiver
// t_col); per edge and tile gH of the receiver (five products on its output
// gradient row) times the filter g (two products), summed on the grid and
// projected once onto the sender's harmonics (no quadrature weights: the
// adjoint of evaluating x on the grid).
template <int U, int NL2, int WPT>
__global__ void __launch_bounds__(64 * (U >= 32 ? U / 32 : 1) * WPT)
    k_gaunt_bwd_send(const int32_t* __restrict__ t_row_ptr, const int32_t* __restrict__ t_perm,
                     const int32_t* __restrict__ t_col, const float* __restrict__ Y,
                     const float* __restrict__ w, const float* __restrict__ gout, float* __restrict__ grad_x,
                     GauntLayout L, const int32_t* __restrict__ order) {
  constexpr int NUT = U >= 32 ? U / 32 : 1;
  constexpr int NW = NUT * WPT, NTH = 64 * NW;
  constexpr int WD = NL2 * U;
  __shared__ __align__(16) float yt[10][kHS];
  __shared__ __align__(16) float hs[NW][32][kHS];
  __shared__ int rs[kChunk], ps_[kChunk];
  __shared__ float ysm[kChunk * 9];
  const int j = order ? min(max(order[blockIdx.x], 0), (int)gridDim.x - 1) : (int)blockIdx.x, t = threadIdx.x;
  const int beg = t_row_ptr[j], end = t_row_ptr[j + 1];
  const int wave = __builtin_amdgcn_readfirstlane(t / 64), lane = t % 64;
  const int ut = wave / WPT, sub = wave % WPT;
  const int n = lane % 32, hk = lane / 32;
  float yv[9];
#pragma unroll
  for (int c = 0; c < 9; ++c) yv[c] = c_grid.y[c][n];
  for (int k = t; k < 9 * kQ; k += NTH) yt[k / kQ][k % kQ] = c_grid.y[k / kQ][k % kQ];
  const int u = 32 * ut + n, uc = u < U ? u : U - 1;
  int oo[5];
  float bp[5];
  out_operand(L, U, uc, hk, n, c_grid.p, oo, bp);
  int wo[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) wo[ks] = (2 * ks + hk < NL2 ? (2 * ks + hk) * U : 0) + uc;
  v16f h, zero;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    h[r] = 0.f;
    zero[r] = 0.f;
  }
  for (int c0 = beg; c0 < end; c0 += kChunk) {
    const int cn = end - c0 < kChunk ? end - c0 : kChunk;
    __syncthreads();
    for (int k = t; k < cn; k += NTH) {
      rs[k] = t_col[c0 + k];
      ps_[k] = t_perm[c0 + k];
    }
    __syncthreads();
    for (int k = t; k < cn * L.ysh; k += NTH)
      ysm[k] = Y[(size_t)ps_[k / L.ysh] * L.ysh + k % L.ysh];
    __syncthreads();
    // edges one at a time, software-pipelined: the next edge's gathers are in
    // flight while this edge's products run (34.5 against 35.9 us)
    struct EdgeOps {
      float ga[5], wa[2];
    };
    // one edge's gathers (the index clamped to the chunk)
    auto fetch = [&](int k, EdgeOps& o) {
      const int kc = k < cn ? k : cn - 1;
      const float* gi = gout + (size_t)rs[kc] * L.outdim;
      const float* we = w + (size_t)ps_[kc] * WD;
#pragma unroll
      for (int ks = 0; ks < 5; ++ks) o.ga[ks] = gi[oo[ks]];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) o.wa[ks] = __builtin_nontemporal_load(we + wo[ks]);
    };
    auto product = [&](int k, const EdgeOps& o) {
      float z[3] = {0.f, 0.f, 0.f};
#pragma unroll
      for (int l2 = 0; l2 < NL2; ++l2)
#pragma unroll
        for (int m = 0; m < 2 * l2 + 1; ++m) z[l2] = fmaf(ysm[k * L.ysh + l2 * l2 + m], yv[l2 * l2 + m], z[l2]);
      const float zb0 = hk ? z[1] : z[0], zb1 = hk ? 0.f : z[2];
      v16f gh = mfma32(o.ga[0], bp[0], zero);
#pragma unroll
      for (int ks = 1; ks < 5; ++ks) gh = mfma32(o.ga[ks], bp[ks], gh);
      v16f g = mfma32(o.wa[0], zb0, zero);
      g = mfma32(o.wa[1], zb1, g);
#pragma unroll
      for (int r = 0; r < 16; ++r) h[r] = fmaf(gh[r], g[r], h[r]);
    };
    if (sub < cn) {
      EdgeOps ea, eb;
      fetch(sub, ea);
      for (int k = sub; k < cn; k += 2 * WPT) {
        fetch(k + WPT, eb);
        __builtin_amdgcn_sched_barrier(0);
        product(k, ea);
        if (k + WPT >= cn) break;
        fetch(k + 2 * WPT, ea);
        __builtin_amdgcn_sched_barrier(0);
        product(k + WPT, eb);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) hs[wave][8 * (r / 4) + 4 * hk + r % 4][n] = h[r];
  __syncthreads();
  if (WPT > 1) {
    for (int k = t; k < NUT * 32 * 32; k += NTH) {
      const int tw = (k / 1024) * WPT, row = (k / 32) % 32, q = k % 32;
      float a = hs[tw][row][q];
#pragma unroll
      for (int s2 = 1; s2 < WPT; ++s2) a += hs[tw + s2][row][q];
      hs[tw][row][q] = a;
    }
    __syncthreads();
  }
  // grad_x[j][block b][uu][m] = sum_q Yq[l_b^2 + m][q] H[uu][q]
  for (int o = t; o < L.xdim; o += NTH) {
    int b = 0;
    while (b + 1 < L.n_in && o >= L.off[b + 1]) ++b;
    const int l = L.deg[b], d = 2 * l + 1, r = o - L.off[b];
    const int uu = r / d, a = l * l + (r - uu * d);
    const float4* hr = reinterpret_cast<const float4*>(hs[(uu / 32) * WPT][uu % 32]);
    const float4* yr = reinterpret_cast<const float4*>(yt[a]);
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < kQ / 4; ++k) {
      const float4 hv = hr[k], yq = yr[k];
      acc = fmaf(hv.x, yq.x, acc);
      acc = fmaf(hv.y, yq.y, acc);
      acc = fmaf(hv.z, yq.z, acc);
      acc = fmaf(hv.w, yq.w, acc);
    }
    grad_x[(size_t)j * L.xdim + o] = acc;
  }
}

// waves per 32-channel tile of the forward: two up to 32 channels (31 against
// 33 us with four and 35 with one on the 1,536-atom graph), else four waves
// per workgroup in all
template <int U>
constexpr int fwd_wpt() {
  return U <= 32 ? 2 : 4 / (U / 32);
}

template <int U>
hipError_t launch(const GauntArgs& a, const GauntLayout& L) {
  constexpr int WPT = fwd_wpt<U>();
  const dim3 blocks(a.n_nodes), threads(64 * (U >= 32 ? U / 32 : 1) * WPT);
  switch (a.lmax_sh) {
    case 0:
      hipLaunchKernelGGL((k_gaunt_conv<U, 1, WPT>), blocks, threads, 0, a.stream, a.row_ptr, a.col, a.x, a.Y,
                         a.w, a.out, L, a.r_order);
      break;
    case 1:
      hipLaunchKernelGGL((k_gaunt_conv<U, 2, WPT>), blocks, threads, 0, a.stream, a.row_ptr, a.col, a.x, a.Y,
                         a.w, a.out, L, a.r_order);
      break;
    default:
      hipLaunchKernelGGL((k_gaunt_conv<U, 3, WPT>), blocks, threads, 0, a.stream, a.row_ptr, a.col, a.x, a.Y,
                         a.w, a.out, L, a.r_order);
      break;
  }
  return hipGetLastError();
}

// waves of the receiver pass (two up to 32 channels: 46 against 50 us with
// four on the 1,536-atom graph), and per 32-channel tile of the sender pass
// (four waves per workgroup in all; two per tile took 36.6 against 34.9 us)
template <int U>
constexpr int recv_waves() {
  return U <= 32 ? 2 : 4;
}
template <int U>
constexpr int send_wpt() {
  return 4 / (U >= 32 ? U / 32 : 1);
}

template <int U, int NL2>
hipError_t launch_bwd_nl(const GauntArgs& a, const GauntLayout& L) {
  constexpr int NW = recv_waves<U>(), WPT = send_wpt<U>();
  const dim3 blocks(a.n_nodes);
  if (a.n_edges > 0 && (a.grad_w || a.grad_Y))
    hipLaunchKernelGGL((k_gaunt_bwd_recv<U, NL2, NW>), blocks, dim3(64 * NW), 0, a.stream, a.row_ptr, a.col,
                       a.x, a.Y, a.w, a.gout, a.grad_Y, a.grad_w, L, a.r_order);
  if (a.grad_x)
    hipLaunchKernelGGL((k_gaunt_bwd_send<U, NL2, WPT>), blocks, dim3(64 * (U >= 32 ? U / 32 : 1) * WPT), 0,
                       a.stream, a.t_row_ptr, a.t_perm, a.t_col, a.Y, a.w, a.gout, a.grad_x, L, a.s_order);
  return hipGetLastError();
}

template <int U>
hipError_t launch_bwd(const GauntArgs& a, const GauntLayout& L) {
  switch (a.lmax_sh) {
    case 0: return launch_bwd_nl<U, 1>(a, L);
    case 1: return launch_bwd_nl<U, 2>(a, L);
    default: return launch_bwd_nl<U, 3>(a, L);
  }
}

}  // namespace

int gaunt_grid_points() { return kQ; }

namespace {
GauntLayout make_layout(const GauntArgs& a) {
  GauntLayout L{};
  L.n_in = a.n_in;
  int off = 0;
  for (int b = 0; b < a.n_in; ++b) {
    L.deg[b] = a.deg[b];
    L.off[b] = off;
    off += a.U * (2 * a.deg[b] + 1);
  }
  L.xdim = off;
  L.ysh = (a.lmax_sh + 1) * (a.lmax_sh + 1);
  L.lout = a.lmax_out;
  L.outdim = a.U * (a.lmax_out + 1) * (a.lmax_out + 1);
  return L;
}
}  // namespace

hipError_t gaunt_forward(const GauntArgs& a) {
  if (a.n_nodes == 0) return hipSuccess;
  const GauntLayout L = make_layout(a);
  switch (a.U) {
    case 16: return launch<16>(a, L);
    case 32: return launch<32>(a, L);
    case 64: return launch<64>(a, L);
    case 128: return launch<128>(a, L);
    default: return hipErrorInvalidValue;
  }
}

hipError_t gaunt_backward(const GauntArgs& a) {
  if (a.n_nodes == 0) return hipSuccess;
  const GauntLayout L = make_layout(a);
  switch (a.U) {
    case 16: return launch_bwd<16>(a, L);
    case 32: return launch_bwd<32>(a, L);
    case 64: return launch_bwd<64>(a, L);
    case 128: return launch_bwd<128>(a, L);
    default: return hipErrorInvalidValue;
  }
}

// ---- second-order backward ---------------------------------------------------
// out is linear in each of x, Y and w, so the gradients of
// L = <gg_x, grad_x> + <gg_Y, grad_Y> + <gg_w, grad_w> are sums of first-order
// results with one operand replaced by its cotangent: per present cotangent
// one forward (its term of d_grad_out) and one backward (its terms of the
// other two gradients).  The first term of each output is written in place,
// later ones go through a scratch row and are added.

namespace {
__global__ void __launch_bounds__(256) k_gaunt_acc(float* __restrict__ y, const float* __restrict__ x,
                                                   long long n) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) y[i] += x[i];
}
__global__ void __launch_bounds__(256) k_gaunt_zero(float* __restrict__ y, long long n) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) y[i] = 0.f;
}
unsigned gaunt_elem_grid(long long n) {
  const long long b = (n + 255) / 256;
  return (unsigned)(b < 4096 ? (b > 0 ? b : 1) : 4096);
}
long long align64(long long n) { return (n + 63) & ~63LL; }   // floats: 256-byte steps

struct GauntAcc {
  float* out;
  float* tmp;
  long long n;
  bool first;
  float* dest() const { return out ? (first ? out : tmp) : nullptr; }
};

// element counts of d_grad_out, d_x, d_Y and d_w
void gaunt_dbl_sizes(const GauntArgs& a, long long (&n)[4]) {
  int xc = 0;
  for (int b = 0; b < a.n_in; ++b) xc += 2 * a.deg[b] + 1;
  n[0] = (long long)a.n_nodes * a.U * (a.lmax_out + 1) * (a.lmax_out + 1);
  n[1] = (long long)a.n_nodes * a.U * xc;
  n[2] = (long long)a.n_edges * (a.lmax_sh + 1) * (a.lmax_sh + 1);
  n[3] = (long long)a.n_edges * (a.lmax_sh + 1) * a.U;
}
}  // namespace

size_t gaunt_double_workspace(const GauntArgs& a) {
  long long n[4];
  gaunt_dbl_sizes(a, n);
  return (size_t)(align64(n[0]) + align64(n[1]) + align64(n[2]) + align64(n[3])) * sizeof(float);
}

hipError_t gaunt_double_backward(const GauntArgs& a, const GauntDbl& d) {
  long long n[4];
  gaunt_dbl_sizes(a, n);
  float* t = static_cast<float*>(d.ws);
  GauntAcc acc[4] = {{d.d_g, t, n[0], true}, {d.d_x, t + align64(n[0]), n[1], true},
                     {d.d_Y, t + align64(n[0]) + align64(n[1]), n[2], true},
                     {d.d_w, t + align64(n[0]) + align64(n[1]) + align64(n[2]), n[3], true}};
  GauntAcc &ag = acc[0], &ax = acc[1], &aY = acc[2], &aw = acc[3];
  auto done = [&](GauntAcc& c) {
    if (!c.out) return;
    if (c.first) {
      c.first = false;
    } else {
      hipLaunchKernelGGL(k_gaunt_acc, dim3(gaunt_elem_grid(c.n)), dim3(256), 0, a.stream, c.out, c.tmp, c.n);
    }
  };
  if (a.n_nodes > 0 && a.n_edges > 0) {
    for (int which = 0; which < 3; ++which) {
      const float* cot = which == 0 ? d.gg_x : which == 1 ? d.gg_Y : d.gg_w;
      if (!cot) continue;
      GauntArgs f = a;
      if (which == 0) f.x = cot;
      if (which == 1) f.Y = cot;
      if (which == 2) f.w = cot;
      if (ag.out) {
        f.out = ag.dest();
        hipError_t e = gaunt_forward(f);
        if (e != hipSuccess) return e;
        done(ag);
      }
      GauntArgs b = f;
      b.out = nullptr;
      b.grad_x = which == 0 ? nullptr : ax.dest();
      b.grad_Y = which == 1 ? nullptr : aY.dest();
      b.grad_w = which == 2 ? nullptr : aw.dest();
      if (b.grad_x || b.grad_Y || b.grad_w) {
        hipError_t e = gaunt_backward(b);
        if (e != hipSuccess) return e;
        if (which != 0) done(ax);
        if (which != 1) done(aY);
        if (which != 2) done(aw);
      }
    }
  }
  // outputs that received no term are zero
  for (GauntAcc& c : acc)
    if (c.out && c.first && c.n > 0)
      hipLaunchKernelGGL(k_gaunt_zero, dim3(gaunt_elem_grid(c.n)), dim3(256), 0, a.stream, c.out, c.n);
  return hipGetLastError();
}

}  // namespace tpc
