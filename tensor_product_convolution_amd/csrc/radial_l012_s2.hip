// Radial-weight kernel specialisations for the 0e+1o+2e / lmax 2 signature.
#include "radial_dbl_kernels.hpp"

namespace tpc {

using SigR = Sig<2, 2, 0, 1, 2>;
constexpr int kNB = 8, kNH = 64;

namespace {

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
constexpr int kRecvWaves = 4;                             // waves per receiver-pass workgroup
int recv_blocks(int n_nodes) {
  const int b = (n_nodes + kRecvWaves - 1) / kRecvWaves;
  return b < 512 ? (b > 0 ? b : 1) : 512;                 // two workgroups per CU
}
int recv_parts(int n_nodes) { return recv_blocks(n_nodes) * kRecvWaves; }
// the second-order receiver pass runs one wave per SIMD: one workgroup per CU
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

}  // namespace

constexpr int kNodeWaves = 4;                             // waves per forward / sender workgroup
// chunk-major grid: (node blocks, chunks); about two workgroups per CU in all
template <int U>
dim3 node_grid(int n_nodes) {
  const int want = (n_nodes + kNodeWaves - 1) / kNodeWaves, cap = 512 / (U / 16);
  return dim3(want < cap ? (want > 0 ? want : 1) : cap, U / 16);
}

// a.geom: a.Y holds the edge vectors r [E][3] and a.grad_Y receives grad_r
template <int U, bool GEOM>
static hipError_t launch_radial_fwd_as(const RadialArgs& a) {
  if (a.n_nodes == 0) return hipSuccess;
  RadialParams rp{a.r_cut, a.W1, a.W2};
  hipLaunchKernelGGL((k_radial_node<SigR, U, kNB, kNH, kNodeWaves, false, GEOM>), node_grid<U>(a.n_nodes),
                     dim3(64 * kNodeWaves), 0, a.stream, a.n_nodes, a.row_ptr, nullptr, a.col, a.x, a.Y,
                     a.r_len, rp, a.out);
  return hipGetLastError();
}
template <int U>
static hipError_t launch_radial_fwd(const RadialArgs& a) {
  return a.geom ? launch_radial_fwd_as<U, true>(a) : launch_radial_fwd_as<U, false>(a);
}

template <int U>
static size_t radial_bwd_ws(int n_nodes, int /*n_edges*/) {
  return align256((size_t)recv_parts(n_nodes) * kNB * kNH * sizeof(float)) +
         (size_t)w2_blocks<U>(n_nodes) * kNH * SigR::NP * U * sizeof(float);
}

// grad_Y and grad_W1 (receiver pass), grad_W2, grad_x (sender pass); a.ws holds
// radial_bwd_ws bytes.  grad_W1/grad_W2/grad_x may be null (skipped).
template <int U, bool GEOM>
static hipError_t launch_radial_bwd_as(const RadialArgs& a) {
  RadialParams rp{a.r_cut, a.W1, a.W2};
  const int nb1 = recv_parts(a.n_nodes), nb2 = w2_blocks<U>(a.n_nodes);
  float* part1 = static_cast<float*>(a.ws);
  float* part2 = reinterpret_cast<float*>(static_cast<char*>(a.ws) +
                                          align256((size_t)nb1 * kNB * kNH * sizeof(float)));
  if (a.grad_Y || a.grad_W1 || a.grad_rlen) {
    hipLaunchKernelGGL((k_radial_bwd_recv<SigR, U, kNB, kNH, kRecvWaves, GEOM>), dim3(recv_blocks(a.n_nodes)),
                       dim3(64 * kRecvWaves), 0, a.stream, a.n_nodes, a.row_ptr, a.col, a.x, a.Y, a.r_len,
                       rp, a.grad_out, a.grad_Y, a.grad_rlen, part1);
    if (a.grad_W1) {
      const long long n = (long long)kNB * kNH;
      hipLaunchKernelGGL(k_radial_sum, dim3((unsigned)((n + 63) / 64)), dim3(64 * kSumWaves), 0, a.stream,
                         part1, nb1, n, a.grad_W1);
    }
  }
  if (a.grad_W2) {
    hipLaunchKernelGGL((k_radial_bwd_w2<SigR, U, kNB, kNH, GEOM>), dim3(nb2, U / 16), dim3(64 * (kNH / 16)), 0,
                       a.stream, a.n_nodes, a.row_ptr, a.col, a.x, a.Y, a.r_len, rp, a.grad_out, part2);
    const long long n = (long long)kNH * SigR::NP * U;
    hipLaunchKernelGGL(k_radial_sum, dim3((unsigned)((n + 63) / 64)), dim3(64 * kSumWaves), 0, a.stream,
                       part2, nb2, n, a.grad_W2);
  }
  if (a.grad_x && a.n_nodes > 0)
    hipLaunchKernelGGL((k_radial_node<SigR, U, kNB, kNH, kNodeWaves, true, GEOM>), node_grid<U>(a.n_nodes),
                       dim3(64 * kNodeWaves), 0, a.stream, a.n_nodes, a.t_row_ptr, a.t_perm, a.t_col,
                       a.grad_out, a.Y, a.r_len, rp, a.grad_x);
  return hipGetLastError();
}

template <int U>
static hipError_t launch_radial_bwd(const RadialArgs& a) {
  return a.geom ? launch_radial_bwd_as<U, true>(a) : launch_radial_bwd_as<U, false>(a);
}

// second-order backward: d_W1 partials (receiver pass), then the two d_W2
// terms' partials, back to back so that one fixed-order sum adds them
template <int U>
static size_t radial_dbl_ws(int n_nodes, int /*n_edges*/) {
  return align256((size_t)dbl_recv_parts(n_nodes) * kNB * kNH * sizeof(float)) +
         (size_t)2 * w2_blocks<U>(n_nodes) * kNH * SigR::NP * U * sizeof(float);
}

// a.grad_out is the unmixed upstream gradient g; a.out receives out_dot (d_g
// before the mix); cotangents a.gg_* may be null (zeros); outputs may be null
template <int U>
static hipError_t launch_radial_dbl(const RadialArgs& a) {
  RadialParams rp{a.r_cut, a.W1, a.W2};
  const int nb1 = dbl_recv_parts(a.n_nodes), nb2 = w2_blocks<U>(a.n_nodes);
  float* part1 = static_cast<float*>(a.ws);
  float* part2 = reinterpret_cast<float*>(static_cast<char*>(a.ws) +
                                          align256((size_t)nb1 * kNB * kNH * sizeof(float)));
  if (a.out && a.n_nodes > 0)
    hipLaunchKernelGGL((k_radial_node_dbl<SigR, U, kNB, kNH, kNodeWaves, false>), node_grid<U>(a.n_nodes),
                       dim3(64 * kNodeWaves), 0, a.stream, a.n_nodes, a.row_ptr, nullptr, a.col, a.x, a.gg_x,
                       a.Y, a.gg_Y, a.r_len, a.gg_rlen, rp, a.out);
  if (a.d_Y || a.d_rlen || a.d_W1) {
    hipLaunchKernelGGL((k_radial_dbl_recv<SigR, U, kNB, kNH, kRecvWaves>), dim3(dbl_recv_blocks(a.n_nodes)),
                       dim3(64 * kRecvWaves), 0, a.stream, a.n_nodes, a.row_ptr, a.col, a.x, a.gg_x, a.Y,
                       a.gg_Y, a.r_len, a.gg_rlen, rp, a.grad_out, a.d_Y, a.d_rlen, part1);
    if (a.d_W1) {
      const long long n = (long long)kNB * kNH;
      hipLaunchKernelGGL(k_radial_sum, dim3((unsigned)((n + 63) / 64)), dim3(64 * kSumWaves), 0, a.stream,
                         part1, nb1, n, a.d_W1);
    }
  }
  if (a.d_W2) {
    const size_t half = (size_t)nb2 * kNH * SigR::NP * U;
    hipLaunchKernelGGL((k_radial_dbl_w2<SigR, U, kNB, kNH, 0>), dim3(nb2, U / 16), dim3(64 * (kNH / 16)), 0,
                       a.stream, a.n_nodes, a.row_ptr, a.col, a.x, a.gg_x, a.Y, a.gg_Y, a.r_len, a.gg_rlen,
                       rp, a.grad_out, part2);
    hipLaunchKernelGGL((k_radial_dbl_w2<SigR, U, kNB, kNH, 1>), dim3(nb2, U / 16), dim3(64 * (kNH / 16)), 0,
                       a.stream, a.n_nodes, a.row_ptr, a.col, a.x, a.gg_x, a.Y, a.gg_Y, a.r_len, a.gg_rlen,
                       rp, a.grad_out, part2 + half);
    const long long n = (long long)kNH * SigR::NP * U;
    hipLaunchKernelGGL(k_radial_sum, dim3((unsigned)((n + 63) / 64)), dim3(64 * kSumWaves), 0, a.stream,
                       part2, 2 * nb2, n, a.d_W2);
  }
  if (a.d_x && a.n_nodes > 0)
    hipLaunchKernelGGL((k_radial_node_dbl<SigR, U, kNB, kNH, kNodeWaves, true>), node_grid<U>(a.n_nodes),
                       dim3(64 * kNodeWaves), 0, a.stream, a.n_nodes, a.t_row_ptr, a.t_perm, a.t_col,
                       a.grad_out, nullptr, a.Y, a.gg_Y, a.r_len, a.gg_rlen, rp, a.d_x);
  return hipGetLastError();
}

template <int U>
static const RadialSet* radial_set() {
  static const RadialSet s{&launch_radial_fwd<U>, &launch_radial_bwd<U>, &radial_bwd_ws<U>,
                           &launch_radial_dbl<U>, &radial_dbl_ws<U>};
  return &s;
}

const RadialSet* radial_l012_s2(int mul, int nb, int nh) {
  if (nb != kNB || nh != kNH) return nullptr;
  switch (mul) {
    case 16: return radial_set<16>();
    case 32: return radial_set<32>();
    case 64: return radial_set<64>();
    case 128: return radial_set<128>();
    default: return nullptr;
  }
}

}  // namespace tpc
