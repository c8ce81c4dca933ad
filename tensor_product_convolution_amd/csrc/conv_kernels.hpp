// Fused tensor-product convolution kernels for gfx950 (wave64).
//
// Forward, one pass per receiver ("Sobek: Streaming Equivariant Tensor
// Product Convolutions", Abstract: edge-local products go straight into
// bounded receiver-side state; "FlashTP", Abstract: fusion, sparsity and all
// paths in one pass):
//   * a workgroup owns one receiver i and streams its CSR segment of edges;
//   * lane -> (edge slot, channel): a wave covers 64/min(U,64) edges at once,
//     each edge on min(U,64) lanes; U > 64 gives each lane U/64 channels;
//   * per edge a lane gathers its channel's x_j components, the edge's Y and
//     its channel's P weights, runs every path's CG nonzeros (compile-time
//     immediates) and accumulates the receiver's output in registers;
//   * the waves' partial sums meet in LDS and the receiver row is stored once,
//     coalesced.  No atomics; the reduction order is fixed, so results are
//     bitwise reproducible.
// Backward:
//   * receiver pass: with grad_out[i] in registers, each edge yields
//     grad_w[e] (per lane) and grad_Y[e] (a butterfly sum over the edge's
//     channel lanes), written once per edge -- these are requested outputs;
//   * sender pass: each workgroup owns a sender j and walks its edges in the
//     sender grouping, gathering grad_out of each receiver, and stores
//     grad_x[j] once.  Again no atomics.
#pragma once
#include "internal.hpp"
#include "sig.hpp"

namespace tpc {

template <int U>
struct LaneMap {
  static_assert(U == 1 || U == 2 || U == 4 || U == 8 || U == 16 || U == 32 || U % 64 == 0,
                "multiplicity must be a power of two up to 64 or a multiple of 64");
  static constexpr int LPE = U >= 64 ? 64 : U;   // lanes per edge
  static constexpr int EPW = 64 / LPE;           // edges per wave step
  static constexpr int CPL = U >= 64 ? U / 64 : 1;  // channels per lane
};

// ---------------------------------------------------------------------------
// per-edge arithmetic of one channel

// out accumulators += sum_p w_p * sum_nz C x_a Y_b
template <class S>
__device__ __forceinline__ void edge_fwd(const float (&xr)[S::XC], const float (&yr)[S::YC],
                                         const float (&wr)[S::NP], float (&acc)[S::OC]) {
  static_for<S::NP>([&](auto P) {
    constexpr PathInfo pi = S::paths.p[P];
    using T = CgPath<pi.l1, pi.l2, pi.l3>;
    constexpr int D3 = 2 * pi.l3 + 1;
    float t[D3];
    static_for<D3>([&](auto C) { t[C] = 0.f; });
    static_for<T::nnz>([&](auto N) {
      constexpr Nz z = T::table.e[N];
      t[z.c] = fmaf(z.v, xr[pi.xo + z.a] * yr[pi.yo + z.b], t[z.c]);
    });
    static_for<D3>([&](auto C) { acc[pi.ko + C] = fmaf(wr[P], t[C], acc[pi.ko + C]); });
  });
}

// grad_w_p = sum_c g_c t_c ; grad_Y_b += sum_p w_p sum_nz C x_a g_c
template <class S>
__device__ __forceinline__ void edge_bwd_recv(const float (&xr)[S::XC], const float (&yr)[S::YC],
                                              const float (&wr)[S::NP], const float (&gr)[S::OC],
                                              float (&gw)[S::NP], float (&gy)[S::YC]) {
  static_for<S::NP>([&](auto P) {
    constexpr PathInfo pi = S::paths.p[P];
    using T = CgPath<pi.l1, pi.l2, pi.l3>;
    constexpr int D3 = 2 * pi.l3 + 1;
    float t[D3];
    static_for<D3>([&](auto C) { t[C] = 0.f; });
    static_for<T::nnz>([&](auto N) {
      constexpr Nz z = T::table.e[N];
      t[z.c] = fmaf(z.v, xr[pi.xo + z.a] * yr[pi.yo + z.b], t[z.c]);
    });
    float s = 0.f;
    static_for<D3>([&](auto C) { s = fmaf(gr[pi.ko + C], t[C], s); });
    gw[P] = s;
    float wg[D3];
    static_for<D3>([&](auto C) { wg[C] = wr[P] * gr[pi.ko + C]; });
    static_for<T::nnz>([&](auto N) {
      constexpr Nz z = T::table.e[N];
      gy[pi.yo + z.b] = fmaf(z.v, xr[pi.xo + z.a] * wg[z.c], gy[pi.yo + z.b]);
    });
  });
}

// grad_x_a += sum_p w_p sum_nz C Y_b g_c
template <class S>
__device__ __forceinline__ void edge_bwd_send(const float (&yr)[S::YC], const float (&wr)[S::NP],
                                              const float (&gr)[S::OC], float (&gx)[S::XC]) {
  static_for<S::NP>([&](auto P) {
    constexpr PathInfo pi = S::paths.p[P];
    using T = CgPath<pi.l1, pi.l2, pi.l3>;
    constexpr int D3 = 2 * pi.l3 + 1;
    float wg[D3];
    static_for<D3>([&](auto C) { wg[C] = wr[P] * gr[pi.ko + C]; });
    static_for<T::nnz>([&](auto N) {
      constexpr Nz z = T::table.e[N];
      gx[pi.xo + z.a] = fmaf(z.v, yr[pi.yo + z.b] * wg[z.c], gx[pi.xo + z.a]);
    });
  });
}

// ---------------------------------------------------------------------------
// row loads of one channel

// x-like row (input irreps): component (irrep i, channel u, a) at U*xoff(i) + u*(2l+1) + a
template <class S, int U>
__device__ __forceinline__ void load_xrow(const float* __restrict__ row, int uu,
                                          float (&v)[LaneMap<U>::CPL][S::XC]) {
  static_for<S::NIN>([&](auto I) {
    constexpr int d = 2 * S::ls.v[I] + 1;
    constexpr int xo = S::xoff(I);
#pragma unroll
    for (int cc = 0; cc < LaneMap<U>::CPL; ++cc) {
      const float* p = row + U * xo + (uu + 64 * cc) * d;
      static_for<d>([&](auto A) { v[cc][xo + A] = p[A]; });
    }
  });
}

// out-like row (output irreps)
template <class S, int U>
__device__ __forceinline__ void load_orow(const float* __restrict__ row, int uu,
                                          float (&v)[LaneMap<U>::CPL][S::OC]) {
  static_for<S::NO>([&](auto K) {
    constexpr OutInfo oi = S::outs.o[K];
    constexpr int d = 2 * oi.l + 1;
#pragma unroll
    for (int cc = 0; cc < LaneMap<U>::CPL; ++cc) {
      const float* p = row + U * oi.ko + (uu + 64 * cc) * d;
      static_for<d>([&](auto C) { v[cc][oi.ko + C] = p[C]; });
    }
  });
}

// ---------------------------------------------------------------------------
// Block reduction of per-lane partial rows and one coalesced store.
// Partial of (wave, channel-set cc, component o, lane) lives at
// red[((wave * CPL + cc) * NC + o) * 65 + lane] (row padded to 65 words).
// Row element t of the stored row decodes to (block, channel u, component).
template <int U, int WPB, int NC, int NB, class Blocks>
__device__ __forceinline__ void block_reduce_store(const float (&v)[LaneMap<U>::CPL][NC],
                                                   float* red, float* __restrict__ dst,
                                                   Blocks) {
  using M = LaneMap<U>;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int cc = 0; cc < M::CPL; ++cc)
#pragma unroll
    for (int o = 0; o < NC; ++o) red[((wv * M::CPL + cc) * NC + o) * 65 + lane] = v[cc][o];
  __syncthreads();
  for (int t = threadIdx.x; t < U * NC; t += WPB * 64) {
    int off = 0, d = 1;
    static_for<NB>([&](auto B) {
      constexpr int bo = Blocks::off(B), bd = Blocks::dim(B);
      if (t >= U * bo) {
        off = bo;
        d = bd;
      }
    });
    const int rem = t - U * off;
    const int u = rem / d;
    const int o = off + (rem - u * d);
    const int cc = M::CPL > 1 ? u / 64 : 0;
    const int uu = u % M::LPE;
    float s = 0.f;
    for (int w2 = 0; w2 < WPB; ++w2)
#pragma unroll
      for (int sl = 0; sl < M::EPW; ++sl) s += red[((w2 * M::CPL + cc) * NC + o) * 65 + sl * M::LPE + uu];
    dst[t] = s;
  }
}

template <class S>
struct OutBlocks {
  static constexpr int off(int k) { return S::outs.o[k].ko; }
  static constexpr int dim(int k) { return 2 * S::outs.o[k].l + 1; }
};
template <class S>
struct InBlocks {
  static constexpr int off(int i) { return S::xoff(i); }
  static constexpr int dim(int i) { return 2 * S::ls.v[i] + 1; }
};

// ---------------------------------------------------------------------------
// kernels

template <class S, int U, int WPB>
__global__ void __launch_bounds__(WPB * 64)
    k_conv_fwd(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col,
               const float* __restrict__ x, const float* __restrict__ Y,
               const float* __restrict__ w, float* __restrict__ out) {
  using M = LaneMap<U>;
  constexpr int XD = U * S::XC, OD = U * S::OC, SLOTS = WPB * M::EPW;
  __shared__ float red[WPB * M::CPL * S::OC * 65];
  const int i = blockIdx.x;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int slot = lane / M::LPE, uu = lane % M::LPE;
  const int beg = row_ptr[i], end = row_ptr[i + 1];
  float acc[M::CPL][S::OC];
#pragma unroll
  for (int cc = 0; cc < M::CPL; ++cc)
#pragma unroll
    for (int o = 0; o < S::OC; ++o) acc[cc][o] = 0.f;
  for (int q = beg + wv * M::EPW + slot; q < end; q += SLOTS) {
    const int j = col[q];
    float xr[M::CPL][S::XC];
    load_xrow<S, U>(x + (size_t)j * XD, uu, xr);
    float yr[S::YC];
#pragma unroll
    for (int b = 0; b < S::YC; ++b) yr[b] = Y[(size_t)q * S::YC + b];
    float wr[M::CPL][S::NP];
#pragma unroll
    for (int p = 0; p < S::NP; ++p)
#pragma unroll
      for (int cc = 0; cc < M::CPL; ++cc) wr[cc][p] = w[((size_t)q * S::NP + p) * U + uu + 64 * cc];
#pragma unroll
    for (int cc = 0; cc < M::CPL; ++cc) edge_fwd<S>(xr[cc], yr, wr[cc], acc[cc]);
  }
  block_reduce_store<U, WPB, S::OC, S::NO>(acc, red, out + (size_t)i * OD, OutBlocks<S>{});
}

template <class S, int U, int WPB>
__global__ void __launch_bounds__(WPB * 64)
    k_conv_bwd_recv(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col,
                    const float* __restrict__ x, const float* __restrict__ Y,
                    const float* __restrict__ w, const float* __restrict__ g,
                    float* __restrict__ grad_w, float* __restrict__ grad_Y) {
  using M = LaneMap<U>;
  constexpr int XD = U * S::XC, OD = U * S::OC, SLOTS = WPB * M::EPW;
  const int i = blockIdx.x;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int slot = lane / M::LPE, uu = lane % M::LPE;
  const int beg = row_ptr[i], end = row_ptr[i + 1];
  if (beg >= end) return;
  float gr[M::CPL][S::OC];
  load_orow<S, U>(g + (size_t)i * OD, uu, gr);
  for (int q = beg + wv * M::EPW + slot; q < end; q += SLOTS) {
    const int j = col[q];
    float xr[M::CPL][S::XC];
    load_xrow<S, U>(x + (size_t)j * XD, uu, xr);
    float yr[S::YC];
#pragma unroll
    for (int b = 0; b < S::YC; ++b) yr[b] = Y[(size_t)q * S::YC + b];
    float wr[M::CPL][S::NP];
#pragma unroll
    for (int p = 0; p < S::NP; ++p)
#pragma unroll
      for (int cc = 0; cc < M::CPL; ++cc) wr[cc][p] = w[((size_t)q * S::NP + p) * U + uu + 64 * cc];
    float gy[S::YC];
#pragma unroll
    for (int b = 0; b < S::YC; ++b) gy[b] = 0.f;
#pragma unroll
    for (int cc = 0; cc < M::CPL; ++cc) {
      float gw[S::NP];
      edge_bwd_recv<S>(xr[cc], yr, wr[cc], gr[cc], gw, gy);
      if (grad_w) {
#pragma unroll
        for (int p = 0; p < S::NP; ++p) grad_w[((size_t)q * S::NP + p) * U + uu + 64 * cc] = gw[p];
      }
    }
    if (grad_Y) {
      // sum over the edge's channel lanes (partners stay inside the slot)
#pragma unroll
      for (int b = 0; b < S::YC; ++b)
#pragma unroll
        for (int off = 1; off < M::LPE; off <<= 1) gy[b] += __shfl_xor(gy[b], off, 64);
      for (int b = uu; b < S::YC; b += M::LPE) {
        float v = 0.f;
#pragma unroll
        for (int bb = 0; bb < S::YC; ++bb)
          if (bb == b) v = gy[bb];
        grad_Y[(size_t)q * S::YC + b] = v;
      }
    }
  }
}

template <class S, int U, int WPB>
__global__ void __launch_bounds__(WPB * 64)
    k_conv_bwd_send(const int32_t* __restrict__ t_row_ptr, const int32_t* __restrict__ t_perm,
                    const int32_t* __restrict__ t_col, const float* __restrict__ Y,
                    const float* __restrict__ w, const float* __restrict__ g,
                    float* __restrict__ grad_x) {
  using M = LaneMap<U>;
  constexpr int XD = U * S::XC, OD = U * S::OC, SLOTS = WPB * M::EPW;
  __shared__ float red[WPB * M::CPL * S::XC * 65];
  const int j = blockIdx.x;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int slot = lane / M::LPE, uu = lane % M::LPE;
  const int beg = t_row_ptr[j], end = t_row_ptr[j + 1];
  float gx[M::CPL][S::XC];
#pragma unroll
  for (int cc = 0; cc < M::CPL; ++cc)
#pragma unroll
    for (int a = 0; a < S::XC; ++a) gx[cc][a] = 0.f;
  for (int k = beg + wv * M::EPW + slot; k < end; k += SLOTS) {
    const int q = t_perm[k];
    const int i = t_col[k];
    float gr[M::CPL][S::OC];
    load_orow<S, U>(g + (size_t)i * OD, uu, gr);
    float yr[S::YC];
#pragma unroll
    for (int b = 0; b < S::YC; ++b) yr[b] = Y[(size_t)q * S::YC + b];
    float wr[M::CPL][S::NP];
#pragma unroll
    for (int p = 0; p < S::NP; ++p)
#pragma unroll
      for (int cc = 0; cc < M::CPL; ++cc) wr[cc][p] = w[((size_t)q * S::NP + p) * U + uu + 64 * cc];
#pragma unroll
    for (int cc = 0; cc < M::CPL; ++cc) edge_bwd_send<S>(yr, wr[cc], gr[cc], gx[cc]);
  }
  block_reduce_store<U, WPB, S::XC, S::NIN>(gx, red, grad_x + (size_t)j * XD, InBlocks<S>{});
}

// ---------------------------------------------------------------------------
// launchers

template <int U>
struct Wpb {
  static constexpr int value = 4;
};

template <class S, int U>
hipError_t launch_fwd(const ConvArgs& a) {
  constexpr int WPB = Wpb<U>::value;
  if (a.n_nodes == 0) return hipSuccess;
  hipLaunchKernelGGL((k_conv_fwd<S, U, WPB>), dim3(a.n_nodes), dim3(WPB * 64), 0, a.stream,
                     a.row_ptr, a.col, a.x, a.Y, a.w, a.out);
  return hipGetLastError();
}

template <class S, int U>
hipError_t launch_bwd_recv(const ConvArgs& a) {
  constexpr int WPB = Wpb<U>::value;
  if (a.n_nodes == 0 || a.n_edges == 0 || (!a.grad_w && !a.grad_Y)) return hipSuccess;
  hipLaunchKernelGGL((k_conv_bwd_recv<S, U, WPB>), dim3(a.n_nodes), dim3(WPB * 64), 0, a.stream,
                     a.row_ptr, a.col, a.x, a.Y, a.w, a.grad_out, a.grad_w, a.grad_Y);
  return hipGetLastError();
}

template <class S, int U>
hipError_t launch_bwd_send(const ConvArgs& a) {
  constexpr int WPB = Wpb<U>::value;
  if (a.n_nodes == 0 || !a.grad_x) return hipSuccess;
  hipLaunchKernelGGL((k_conv_bwd_send<S, U, WPB>), dim3(a.n_nodes), dim3(WPB * 64), 0, a.stream,
                     a.t_row_ptr, a.t_perm, a.t_col, a.Y, a.w, a.grad_out, a.grad_x);
  return hipGetLastError();
}

template <class S, int U>
const KernelSet* kernel_set() {
  static const KernelSet k{&launch_fwd<S, U>, &launch_bwd_recv<S, U>, &launch_bwd_send<S, U>};
  return &k;
}

}  // namespace tpc
