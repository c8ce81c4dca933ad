// Launch sequences of the radial-weight kernels, shared by the signature units
// (radial_l012_s2.hip, radial_l0123_s3.hip).  Everything here has internal
// linkage: each unit instantiates it for its own signature.
#pragma once
#include "radial_dbl_kernels.hpp"

namespace tpc {
namespace {

constexpr int kNB = 8, kNH = 64;                          // basis functions, hidden units

// out[e] = sum_b part[b][e] in a fixed order: lane = element (64 per
// workgroup); wave w sums the partials b = w, w + kSumWaves, ... in order with
// eight loads in flight, and the wave sums are added in wave order.  (One
// thread per element summing all partials in turn took 0.38 ms for the 512
// grad_W1 elements over 2,048 partials: a chain of dependent loads.)
constexpr int kSumWaves = 16;
__global__ void __launch_bounds__(64 * kSumWaves)
    k_radial_sum(const float* __restrict__ part, int nparts, long long n, float* __restrict__ out) {
  __shared__ float red[kSumWaves][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const long long e = (long long)blockIdx.x * 64 + lane;
  const long long ec = e < n ? e : n - 1;
  float s = 0.f;
  int b = wv;
  for (; b + 7 * kSumWaves < nparts; b += 8 * kSumWaves) {
    float q[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = part[(size_t)(b + j * kSumWaves) * n + ec];
#pragma unroll
    for (int j = 0; j < 8; ++j) s += q[j];
  }
  for (; b < nparts; b += kSumWaves) s += part[(size_t)b * n + ec];
  red[wv][lane] = s;
  __syncthreads();
  if (wv == 0 && e < n) {
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < kSumWaves; ++w) a += red[w][lane];
    out[e] = a;
  }
}

// persistent grid sizes (fixed functions of the node count, so the partial
// sums and hence the results do not depend on the device)
template <int NW>                                         // NW waves per receiver-pass workgroup
int recv_blocks(int n_nodes) {
  const int b = (n_nodes + NW - 1) / NW;
  return b < 512 ? (b > 0 ? b : 1) : 512;
}
template <int NW>
int recv_parts(int n_nodes) { return recv_blocks<NW>(n_nodes) * NW; }
// the second-order receiver pass runs one wave per SIMD: one workgroup of
// kRecvWaves per CU
constexpr int kRecvWaves = 4;
int dbl_recv_blocks(int n_nodes) {
  const int b = (n_nodes + kRecvWaves - 1) / kRecvWaves;
  return b < 256 ? (b > 0 ? b : 1) : 256;
}
int dbl_recv_parts(int n_nodes) { return dbl_recv_blocks(n_nodes) * kRecvWaves; }
template <int U>
int w2_blocks(int n_nodes) {
  const int want = (n_nodes + kNH / 16 - 1) / (kNH / 16), cap = 512 / (U / 16);
  return want < cap ? (want > 0 ? want : 1) : cap;
}

size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

constexpr int kNodeWaves = 4;                             // waves per forward / sender workgroup
// chunk-major grid: (node blocks, chunks); about two workgroups per CU in all.
// node_grid: a node per wave at a time (second-order passes); group_grid: a
// node per 16-lane group (k_radial_node), four per wave
template <int U>
dim3 node_grid(int n_nodes) {
  const int want = (n_nodes + kNodeWaves - 1) / kNodeWaves, cap = 512 / (U / 16);
  return dim3(want < cap ? (want > 0 ? want : 1) : cap, U / 16);
}
template <int U>
dim3 group_grid(int n_nodes) {
  const int want = (n_nodes + 4 * kNodeWaves - 1) / (4 * kNodeWaves), cap = 512 / (U / 16);
  return dim3(want < cap ? (want > 0 ? want : 1) : cap, U / 16);
}

// A signature's radial kernels: S the CG signature, NPG the paths per grad_W2
// launch (the grad_w tile of NPG paths must fit in LDS), RW the waves of a
// receiver-pass workgroup, DBL whether the second-order kernels are built for
// it.
template <class S, int NPG, int RW, bool DBL>
struct RadialSig {
  using Sig = S;
  static constexpr int npg = NPG;
  static constexpr int recv_waves = RW;
  static constexpr bool dbl = DBL;
};

// a.geom: a.Y holds the edge vectors r [E][3] and a.grad_Y receives grad_r
template <class R, int U, bool GEOM>
hipError_t launch_radial_fwd_as(const RadialArgs& a) {
  using S = typename R::Sig;
  if (a.n_nodes == 0) return hipSuccess;
  RadialParams rp{a.r_cut, a.W1, a.W2};
  hipLaunchKernelGGL((k_radial_node<S, U, kNB, kNH, kNodeWaves, false, GEOM>), group_grid<U>(a.n_nodes),
                     dim3(64 * kNodeWaves), 0, a.stream, a.n_nodes, a.row_ptr, nullptr, a.col, a.x, a.Y,
                     a.r_len, rp, a.out, a.r_order);
  return hipGetLastError();
}
template <class R, int U>
hipError_t launch_radial_fwd(const RadialArgs& a) {
  return a.geom ? launch_radial_fwd_as<R, U, true>(a) : launch_radial_fwd_as<R, U, false>(a);
}

template <class R, int U>
size_t radial_bwd_ws(int n_nodes, int /*n_edges*/) {
  return align256((size_t)recv_parts<R::recv_waves>(n_nodes) * kNB * kNH * sizeof(float)) +
         (size_t)w2_blocks<U>(n_nodes) * kNH * R::Sig::NP * U * sizeof(float);
}

// the grad_W2 partials, one launch per path group G (paths G*NPG ..)
template <class R, int U, bool GEOM, int G = 0>
void launch_w2_groups(const RadialArgs& a, const RadialParams& rp, int nb2, float* part2) {
  using S = typename R::Sig;
  constexpr int P0 = G * R::npg;
  if constexpr (P0 < S::NP) {
    constexpr int N = S::NP - P0 < R::npg ? S::NP - P0 : R::npg;
    hipLaunchKernelGGL((k_radial_bwd_w2<S, U, kNB, kNH, GEOM, P0, N>), dim3(nb2, U / 16), dim3(64 * (kNH / 16)),
                       0, a.stream, a.n_nodes, a.row_ptr, a.col, a.x, a.Y, a.r_len, rp, a.grad_out, part2,
                       a.r_order);
    launch_w2_groups<R, U, GEOM, G + 1>(a, rp, nb2, part2);
  }
}

// grad_Y and grad_W1 (receiver pass), grad_W2, grad_x (sender pass); a.ws holds
// radial_bwd_ws bytes.  grad_W1/grad_W2/grad_x may be null (skipped).
template <class R, int U, bool GEOM>
hipError_t launch_radial_bwd_as(const RadialArgs& a) {
  using S = typename R::Sig;
  constexpr int RW = R::recv_waves;
  RadialParams rp{a.r_cut, a.W1, a.W2};
  const int nb1 = recv_parts<RW>(a.n_nodes), nb2 = w2_blocks<U>(a.n_nodes);
  float* part1 = static_cast<float*>(a.ws);
  float* part2 = reinterpret_cast<float*>(static_cast<char*>(a.ws) +
                                          align256((size_t)nb1 * kNB * kNH * sizeof(float)));
  if (a.grad_Y || a.grad_W1 || a.grad_rlen) {
    hipLaunchKernelGGL((k_radial_bwd_recv<S, U, kNB, kNH, RW, GEOM>), dim3(recv_blocks<RW>(a.n_nodes)),
                       dim3(64 * RW), 0, a.stream, a.n_nodes, a.row_ptr, a.col, a.x, a.Y, a.r_len,
                       rp, a.grad_out, a.grad_Y, a.grad_rlen, part1, a.r_order);
    if (a.grad_W1) {
      const long long n = (long long)kNB * kNH;
      hipLaunchKernelGGL(k_radial_sum, dim3((unsigned)((n + 63) / 64)), dim3(64 * kSumWaves), 0, a.stream,
                         part1, nb1, n, a.grad_W1);
    }
  }
  if (a.grad_W2) {
    launch_w2_groups<R, U, GEOM>(a, rp, nb2, part2);
    const long long n = (long long)kNH * S::NP * U;
    hipLaunchKernelGGL(k_radial_sum, dim3((unsigned)((n + 63) / 64)), dim3(64 * kSumWaves), 0, a.stream,
                       part2, nb2, n, a.grad_W2);
  }
  if (a.grad_x && a.n_nodes > 0)
    hipLaunchKernelGGL((k_radial_node<S, U, kNB, kNH, kNodeWaves, true, GEOM>), group_grid<U>(a.n_nodes),
                       dim3(64 * kNodeWaves), 0, a.stream, a.n_nodes, a.t_row_ptr, a.t_perm, a.t_col,
                       a.grad_out, a.Y, a.r_len, rp, a.grad_x, a.s_order);
  return hipGetLastError();
}

template <class R, int U>
hipError_t launch_radial_bwd(const RadialArgs& a) {
  return a.geom ? launch_radial_bwd_as<R, U, true>(a) : launch_radial_bwd_as<R, U, false>(a);
}

// second-order backward: d_W1 partials (receiver pass), then the two d_W2
// terms' partials, back to back so that one fixed-order sum adds them
template <class R, int U>
size_t radial_dbl_ws(int n_nodes, int /*n_edges*/) {
  return align256((size_t)dbl_recv_parts(n_nodes) * kNB * kNH * sizeof(float)) +
         (size_t)2 * w2_blocks<U>(n_nodes) * kNH * R::Sig::NP * U * sizeof(float);
}

// the two d_W2 terms' partials, one launch per term and path group
template <class R, int U, int KIND, int G = 0>
void launch_dbl_w2_groups(const RadialArgs& a, const RadialParams& rp, int nb2, float* part2) {
  using S = typename R::Sig;
  constexpr int P0 = G * R::npg;
  if constexpr (P0 < S::NP) {
    constexpr int N = S::NP - P0 < R::npg ? S::NP - P0 : R::npg;
    hipLaunchKernelGGL((k_radial_dbl_w2<S, U, kNB, kNH, KIND, P0, N>), dim3(nb2, U / 16), dim3(64 * (kNH / 16)),
                       0, a.stream, a.n_nodes, a.row_ptr, a.col, a.x, a.gg_x, a.Y, a.gg_Y, a.r_len, a.gg_rlen,
                       rp, a.grad_out, part2, a.r_order);
    launch_dbl_w2_groups<R, U, KIND, G + 1>(a, rp, nb2, part2);
  }
}

// a.grad_out is the unmixed upstream gradient g; a.out receives out_dot (d_g
// before the mix); cotangents a.gg_* may be null (zeros); outputs may be null
template <class R, int U>
hipError_t launch_radial_dbl(const RadialArgs& a) {
  using S = typename R::Sig;
  RadialParams rp{a.r_cut, a.W1, a.W2};
  const int nb1 = dbl_recv_parts(a.n_nodes), nb2 = w2_blocks<U>(a.n_nodes);
  float* part1 = static_cast<float*>(a.ws);
  float* part2 = reinterpret_cast<float*>(static_cast<char*>(a.ws) +
                                          align256((size_t)nb1 * kNB * kNH * sizeof(float)));
  if (a.out && a.n_nodes > 0)
    hipLaunchKernelGGL((k_radial_node_dbl<S, U, kNB, kNH, kNodeWaves, false>), node_grid<U>(a.n_nodes),
                       dim3(64 * kNodeWaves), 0, a.stream, a.n_nodes, a.row_ptr, nullptr, a.col, a.x, a.gg_x,
                       a.Y, a.gg_Y, a.r_len, a.gg_rlen, rp, a.out, a.r_order);
  if (a.d_Y || a.d_rlen || a.d_W1) {
    hipLaunchKernelGGL((k_radial_dbl_recv<S, U, kNB, kNH, kRecvWaves>), dim3(dbl_recv_blocks(a.n_nodes)),
                       dim3(64 * kRecvWaves), 0, a.stream, a.n_nodes, a.row_ptr, a.col, a.x, a.gg_x, a.Y,
                       a.gg_Y, a.r_len, a.gg_rlen, rp, a.grad_out, a.d_Y, a.d_rlen, part1, a.r_order);
    if (a.d_W1) {
      const long long n = (long long)kNB * kNH;
      hipLaunchKernelGGL(k_radial_sum, dim3((unsigned)((n + 63) / 64)), dim3(64 * kSumWaves), 0, a.stream,
                         part1, nb1, n, a.d_W1);
    }
  }
  if (a.d_W2) {
    const size_t half = (size_t)nb2 * kNH * S::NP * U;
    launch_dbl_w2_groups<R, U, 0>(a, rp, nb2, part2);
    launch_dbl_w2_groups<R, U, 1>(a, rp, nb2, part2 + half);
    const long long n = (long long)kNH * S::NP * U;
    hipLaunchKernelGGL(k_radial_sum, dim3((unsigned)((n + 63) / 64)), dim3(64 * kSumWaves), 0, a.stream,
                       part2, 2 * nb2, n, a.d_W2);
  }
  if (a.d_x && a.n_nodes > 0)
    hipLaunchKernelGGL((k_radial_node_dbl<S, U, kNB, kNH, kNodeWaves, true>), node_grid<U>(a.n_nodes),
                       dim3(64 * kNodeWaves), 0, a.stream, a.n_nodes, a.t_row_ptr, a.t_perm, a.t_col,
                       a.grad_out, nullptr, a.Y, a.gg_Y, a.r_len, a.gg_rlen, rp, a.d_x, a.s_order);
  return hipGetLastError();
}

template <class R, int U>
const RadialSet* radial_set() {
  if constexpr (R::dbl) {
    static const RadialSet s{&launch_radial_fwd<R, U>, &launch_radial_bwd<R, U>, &radial_bwd_ws<R, U>,
                             &launch_radial_dbl<R, U>, &radial_dbl_ws<R, U>};
    return &s;
  } else {
    static const RadialSet s{&launch_radial_fwd<R, U>, &launch_radial_bwd<R, U>, &radial_bwd_ws<R, U>, nullptr,
                             nullptr};
    return &s;
  }
}

}  // namespace
}  // namespace tpc
