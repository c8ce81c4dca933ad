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
// Workgroup = one receiver, 4 waves; U <= 32: the waves split the receiver's
// edges; U = 64 / 128: two / four 32-channel tiles, the waves of a tile split
// the edges.  The waves meet in LDS, the projection onto the output harmonics
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
constexpr int kBatch = 8;     // edges whose gathers one wave has in flight together
constexpr int kChunk = 256;   // edges whose sender index and Y row are staged in LDS at a time

typedef float v16f __attribute__((ext_vector_type(16)));

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
template <int U, int NL2>
__global__ void __launch_bounds__(256)
    k_gaunt_conv(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col,
                 const float* __restrict__ x, const float* __restrict__ Y, const float* __restrict__ w,
                 float* __restrict__ out, GauntLayout L) {
  constexpr int NUT = U >= 32 ? U / 32 : 1;       // 32-channel tiles
  constexpr int WPT = 4 / NUT;                    // waves per tile
  constexpr int WD = NL2 * U;                     // weights per edge
  __shared__ __align__(16) float ps[9][kHS];
  __shared__ __align__(16) float hs[4][32][kHS];
  __shared__ int cs[kChunk];
  __shared__ float ysm[kChunk * 9];
  const int i = blockIdx.x, t = threadIdx.x;
  const int beg = row_ptr[i], end = row_ptr[i + 1];
  const int wave = __builtin_amdgcn_readfirstlane(t / 64), lane = t % 64;
  const int ut = wave / WPT, sub = wave % WPT;
  const int n = lane % 32, hk = lane / 32;
  float yv[9];
#pragma unroll
  for (int c = 0; c < 9; ++c) yv[c] = c_grid.y[c][n];      // harmonics at this lane's point
  for (int k = t; k < 9 * kQ; k += 256) ps[k / kQ][k % kQ] = c_grid.p[k / kQ][k % kQ];
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
  // kChunk edges); each wave walks its edges (wave-uniform) two at a time with
  // two operand buffers, so one edge's gathers are in flight while the other's
  // products run.  Every fetch is issued (the index is clamped to the chunk)
  // so the number of loads in flight is the same on every path.
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
    for (int k = t; k < cn; k += 256) cs[k] = col[c0 + k];
    for (int k = t; k < cn * L.ysh; k += 256) ysm[k] = Y[(size_t)c0 * L.ysh + k];
    __syncthreads();
    // batches of kBatch edges per wave: all gathers of a batch are issued
    // before its products, which then wait for their own loads only (loads
    // complete in order).  Slots past the chunk's end re-read its last edge and
    // are multiplied by zero (straight-line code keeps every load up front).
    for (int k0 = sub; k0 < cn; k0 += kBatch * WPT) {
      Ops o[kBatch];
#pragma unroll
      for (int r = 0; r < kBatch; ++r) fetch(c0, k0 + r * WPT < cn ? k0 + r * WPT : cn - 1, o[r]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < kBatch; r += 2) {
        const bool ok0 = k0 + r * WPT < cn, ok1 = k0 + (r + 1) * WPT < cn;
        product2(o[r], ok0 ? k0 + r * WPT : cn - 1, ok0 ? 1.f : 0.f, o[r + 1],
                 ok1 ? k0 + (r + 1) * WPT : cn - 1, ok1 ? 1.f : 0.f);
      }
    }
  }
  // D[row][col = q]: row = 8 (r / 4) + 4 hk + r % 4 (channel within the tile)
#pragma unroll
  for (int r = 0; r < 16; ++r) hs[wave][8 * (r / 4) + 4 * hk + r % 4][n] = h[r];
  __syncthreads();
  if (WPT > 1) {   // the waves of a tile add up, once, into the tile's first copy
    for (int k = t; k < NUT * 32 * 32; k += 256) {
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
  for (int o = t; o < L.outdim; o += 256) {
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

template <int U>
hipError_t launch(const GauntArgs& a, const GauntLayout& L) {
  const dim3 blocks(a.n_nodes), threads(256);
  switch (a.lmax_sh) {
    case 0:
      hipLaunchKernelGGL((k_gaunt_conv<U, 1>), blocks, threads, 0, a.stream, a.row_ptr, a.col, a.x, a.Y, a.w,
                         a.out, L);
      break;
    case 1:
      hipLaunchKernelGGL((k_gaunt_conv<U, 2>), blocks, threads, 0, a.stream, a.row_ptr, a.col, a.x, a.Y, a.w,
                         a.out, L);
      break;
    default:
      hipLaunchKernelGGL((k_gaunt_conv<U, 3>), blocks, threads, 0, a.stream, a.row_ptr, a.col, a.x, a.Y, a.w,
                         a.out, L);
      break;
  }
  return hipGetLastError();
}

}  // namespace

int gaunt_grid_points() { return kQ; }

hipError_t gaunt_forward(const GauntArgs& a) {
  if (a.n_nodes == 0) return hipSuccess;
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
  switch (a.U) {
    case 16: return launch<16>(a, L);
    case 32: return launch<32>(a, L);
    case 64: return launch<64>(a, L);
    case 128: return launch<128>(a, L);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tpc
