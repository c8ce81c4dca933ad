// Convolution with fully connected per-edge weights, by reassociation
// ("Sobek: Streaming Equivariant Tensor Product Convolutions", Abstract:
// radial projection, harmonic coupling and aggregation are reassociated so
// that edge-local products go straight into bounded receiver-side state;
// fully connected multiplicity mixing is preserved).
//
//   W_e[p, u, v] = sum_h R_e[h] Theta[h, p, u, v]          (never formed)
//   out[i, k, v, c] = sum_{e into i} sum_{p->k} sum_u W_e[p, u, v] T_p(x_j[u], Y_e)[c]
//                   = sum_{h, p->k, u} Theta[h, p, u, v] S_i[h, p, u, c]
//   S_i[h, p, u, c] = sum_{e into i} R_e[h] T_p(x_j[u], Y_e)[c]
//
// Phase 1 (k_fc_state) streams each receiver's edges into S_i: per 16-edge
// tile the lanes form the CG terms T of their edges (VALU, compile-time
// nonzeros) and MFMA accumulates R^T T (M = hidden units, N = 16 channels,
// K = edges).  S is node-sized (no edge-sized array is written) and is laid
// out per output irrep k as rows (i, c) of length K_k = H |P_k| U, ordered
// (h, path of k, u).  Phase 2 (k_fc_contract) is then a dense product per
// irrep, out_k[(i,c)][v] = sum_K S_k[(i,c)][K] Theta_k[K][v], on MFMA.
// MFMA operand layout (16x16x4 f32, wave64): lane l supplies A[l%16][l/16],
// B[l/16][l%16] and holds D[4(l/16)+i][l%16].
#include "radial_kernels.hpp"

namespace tpc {

// per-plan constants of the state layout (host-filled)
struct FcLayout {
  int n_out;                  // output irreps
  long long base[8];          // float offset of S_k
  int d3[8], npk[8], ko[8];   // 2l+1, paths into k, per-channel output offset
  int pg[8][8];               // global path index of the p-th path into k
};

namespace {

// position of path P among the paths into its output irrep
template <class S>
constexpr int path_local(int p) {
  int n = 0;
  for (int q = 0; q < p; ++q)
    if (S::paths.p[q].k == S::paths.p[p].k) ++n;
  return n;
}
template <class S>
constexpr int paths_into(int k) {
  int n = 0;
  for (int q = 0; q < S::NP; ++q)
    if (S::paths.p[q].k == k) ++n;
  return n;
}
// output components of paths [P0, P0 + N)
template <class S>
constexpr int comps(int p0, int n) {
  int t = 0;
  for (int q = p0; q < p0 + n; ++q) t += 2 * S::paths.p[q].l3 + 1;
  return t;
}
template <class S>
constexpr int comp_off(int p0, int p) { return comps<S>(p0, p - p0); }

// Phase 1.  One workgroup (4 waves) per receiver; wave w takes channel chunk
// w % NCH and path group w / NCH.
template <class S, int U, int H>
__global__ void __launch_bounds__(256)
    k_fc_state(int n_nodes, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col,
               const float* __restrict__ x, const float* __restrict__ Y, const float* __restrict__ R,
               float* __restrict__ Sbuf, FcLayout lay) {
  constexpr int NCH = U / 16, NGRP = 4 / NCH, PPG = (S::NP + NGRP - 1) / NGRP;
  static_assert(NCH * NGRP == 4 && H <= 16, "fc tiling");
  const int i = blockIdx.x;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int e16 = lane & 15, g = lane >> 4;
  const int ch = wv % NCH, grp = wv / NCH;
  const int u = 16 * ch + e16;
  const int beg = row_ptr[i], end = row_ptr[i + 1];
  static_for<NGRP>([&](auto G) {
    if (grp != G) return;
    constexpr int P0 = G * PPG;
    constexpr int NPP = S::NP - P0 < PPG ? S::NP - P0 : PPG;
    constexpr int NT = comps<S>(P0, NPP);          // (path, component) tiles of this wave
    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int t0 = beg; t0 < end; t0 += 16) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int q = t0 + 4 * g + r;
        const bool v = q < end;
        const int qc = v ? q : end - 1;
        // A: R[edge 4g + r][h = l%16] (zero rows past H and for a padded edge)
        const float a = (v && e16 < H) ? R[(size_t)qc * H + e16] : 0.f;
        float xr[S::XC], yr[S::YC];
        load_x_channel<S, U>(x, col[qc], u, xr);
#pragma unroll
        for (int b = 0; b < S::YC; ++b) yr[b] = Y[(size_t)qc * S::YC + b];
        // B: the CG terms of this edge and channel, one per (path, component)
        float tv[NT];
        static_for<NPP>([&](auto PP) {
          constexpr PathInfo pi = S::paths.p[P0 + PP];
          using T = CgPath<pi.l1, pi.l2, pi.l3>;
          constexpr int D3 = 2 * pi.l3 + 1, OFF = comp_off<S>(P0, P0 + PP);
          static_for<D3>([&](auto C) { tv[OFF + C] = 0.f; });
          static_for<T::nnz>([&](auto N) {
            constexpr Nz z = T::table.e[N];
            tv[OFF + z.c] = fmaf(z.v, xr[pi.xo + z.a] * yr[pi.yo + z.b], tv[OFF + z.c]);
          });
        });
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = mfma_16x16x4(a, tv[t], acc[t]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // S_k[(i, c)][(h, path of k, u)]: lane holds rows h = 4(l/16) + r of column u
    if (g * 4 < H) {
      static_for<NPP>([&](auto PP) {
        constexpr int P = P0 + PP;
        constexpr PathInfo pi = S::paths.p[P];
        constexpr int D3 = 2 * pi.l3 + 1, OFF = comp_off<S>(P0, P);
        constexpr int NPK = paths_into<S>(pi.k), PL = path_local<S>(P);
        constexpr int KK = H * NPK * U;
        float* Sk = Sbuf + lay.base[pi.k] + (size_t)i * D3 * KK;
        static_for<D3>([&](auto C) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int h = 4 * g + r;
            if (h < H) Sk[(size_t)C * KK + (size_t)(h * NPK + PL) * U + u] = acc[OFF + C][r];
          }
        });
      });
    }
  });
}

// Phase 2.  One workgroup (4 waves) per tile of 16 rows (i, c) of one output
// irrep; the waves split the contraction length K_k in four and meet in LDS.
// Within a wave, lane group l/16 takes four consecutive K per four MFMA steps
// (the order of a sum over K is free), so each lane reads its row with one
// 16-byte load per four steps.  Rows of all irreps are enumerated irrep by
// irrep (blockIdx.x).
template <int U, int H>
__global__ void __launch_bounds__(256)
    k_fc_contract(int n_nodes, const float* __restrict__ Sbuf, const float* __restrict__ Theta, int P,
                  int outdim, float* __restrict__ out, FcLayout lay) {
  constexpr int NV = U / 16;
  __shared__ float red[3][NV][4][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int e16 = lane & 15, g = lane >> 4;
  int k = 0, first = 0;
  while (k + 1 < lay.n_out && (int)blockIdx.x >= first + (n_nodes * lay.d3[k] + 15) / 16) {
    first += (n_nodes * lay.d3[k] + 15) / 16;
    ++k;
  }
  const int d3 = lay.d3[k], npk = lay.npk[k];
  const int KK = H * npk * U;                       // a multiple of 256
  const int rows = n_nodes * d3;
  const int row0 = ((int)blockIdx.x - first) * 16;
  const int ra = row0 + e16;                         // this lane's A row
  const bool va = ra < rows;
  const float* arow = Sbuf + lay.base[k] + (size_t)(va ? ra : rows - 1) * KK;
  const int kq = KK / 4;                             // this wave's share of K
  const int K0 = wv * kq;
  f32x4 acc[NV];
#pragma unroll
  for (int n = 0; n < NV; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  // K = (h * npk + pl) * U + uu; a 16-aligned block of K shares (h, pl), so
  // t = K / U is uniform over the wave and Theta's row block is a scalar base.
  for (int t = K0 / U; t < (K0 + kq) / U; ++t) {
    const int pl = t % npk, h = t / npk;
    const float* thb = Theta + ((size_t)h * P + lay.pg[k][pl]) * U * U + e16;
    const float* ab = arow + (size_t)t * U + 4 * g;
#pragma unroll
    for (int ub = 0; ub < U; ub += 16) {
      const float4 a4 = va ? *reinterpret_cast<const float4*>(ab + ub) : float4{0.f, 0.f, 0.f, 0.f};
      const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const float* th = thb + (size_t)(ub + 4 * g + st) * U;
#pragma unroll
        for (int n = 0; n < NV; ++n) acc[n] = mfma_16x16x4(av[st], th[16 * n], acc[n]);
      }
    }
  }
  if (wv > 0) {
#pragma unroll
    for (int n = 0; n < NV; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wv - 1][n][r][lane] = acc[n][r];
  }
  __syncthreads();
  if (wv == 0) {
#pragma unroll
    for (int n = 0; n < NV; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[n][r] += red[0][n][r][lane] + red[1][n][r][lane] + red[2][n][r][lane];
    // D[row 4g + r][v = 16n + l%16]
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = row0 + 4 * g + r;
      if (row < rows) {
        const int node = row / d3, c = row - node * d3;
        float* o = out + (size_t)node * outdim + (size_t)U * lay.ko[k] + c;
#pragma unroll
        for (int n = 0; n < NV; ++n) o[(size_t)(16 * n + e16) * d3] = acc[n][r];
      }
    }
  }
}

using SigF = Sig<2, 2, 0, 1, 2>;
constexpr int kH = 8;

template <int U>
FcLayout make_layout(int n_nodes) {
  FcLayout L{};
  L.n_out = SigF::NO;
  long long off = 0;
  for (int k = 0; k < SigF::NO; ++k) {
    L.d3[k] = 2 * SigF::outs.o[k].l + 1;
    L.ko[k] = SigF::outs.o[k].ko;
    int n = 0;
    for (int p = 0; p < SigF::NP; ++p)
      if (SigF::paths.p[p].k == k) L.pg[k][n++] = p;
    L.npk[k] = n;
    L.base[k] = off;
    off += (long long)n_nodes * L.d3[k] * kH * n * U;
  }
  return L;
}

template <int U>
size_t fc_ws(int n_nodes) {
  const FcLayout L = make_layout<U>(n_nodes);
  long long tot = 0;
  for (int k = 0; k < L.n_out; ++k) tot += (long long)n_nodes * L.d3[k] * kH * L.npk[k] * U;
  return (size_t)tot * sizeof(float);
}

template <int U>
hipError_t launch_fc_fwd(const FcArgs& a) {
  if (a.n_nodes == 0) return hipSuccess;
  const FcLayout L = make_layout<U>(a.n_nodes);
  float* Sbuf = static_cast<float*>(a.ws);
  hipLaunchKernelGGL((k_fc_state<SigF, U, kH>), dim3(a.n_nodes), dim3(256), 0, a.stream, a.n_nodes, a.row_ptr,
                     a.col, a.x, a.Y, a.R, Sbuf, L);
  int tiles = 0;
  for (int k = 0; k < L.n_out; ++k) tiles += (a.n_nodes * L.d3[k] + 15) / 16;
  hipLaunchKernelGGL((k_fc_contract<U, kH>), dim3(tiles), dim3(256), 0, a.stream, a.n_nodes, Sbuf, a.Theta,
                     SigF::NP, a.outdim, a.out, L);
  return hipGetLastError();
}

template <int U>
const FcSet* fc_set() {
  static const FcSet s{&launch_fc_fwd<U>, &fc_ws<U>, kH};
  return &s;
}

}  // namespace

const FcSet* fc_l012_s2(int mul, int n_radial) {
  if (n_radial != kH) return nullptr;
  switch (mul) {
    case 16: return fc_set<16>();
    case 32: return fc_set<32>();
    default: return nullptr;
  }
}

}  // namespace tpc
