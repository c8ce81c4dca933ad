// Second-order backward of the convolution ("Sobek: Streaming Equivariant
// Tensor Product Convolutions", Abstract: forward, backward and double
// backward).  With F(g, x, Y, w) = <g, out(x, Y, w)>, linear in each argument,
// the first backward returns grad F = (gx, gY, gw).  For cotangents (ggx, ggY,
// ggw) of those, L = <ggx, gx> + <ggY, gY> + <ggw, gw> equals
// F(g, ggx, Y, w) + F(g, x, ggY, w) + F(g, x, Y, ggw), hence
//   dg = out(ggx, Y, w) + out(x, ggY, w) + out(x, Y, ggw)      receiver-side
//   dY = gY(ggx, w, g) + gY(x, ggw, g)                          per edge
//   dw = gw(ggx, Y, g) + gw(x, ggY, g)                          per edge
//   dx = gx(ggY, w, g) + gx(Y, ggw, g)                          sender-side
// Every term is the per-lane arithmetic of a first-order pass with one
// operand replaced, so one receiver-grouped pass produces dg, dY and dw (the
// Z-form of x against g serves both the ggY and the ggw term) and one
// sender-grouped pass produces dx.  A missing cotangent counts as zero.
// Lane map as in the first-order kernels (LaneMap): lanes = (edge slot,
// channel), one or four waves per node; operands are read straight from
// global memory.
#pragma once

namespace tpc {

// sum over the edge slots of the wave (lane bits at and above LPE)
template <int LPE, int N>
__device__ __forceinline__ void cross_slot_sum(float (&v)[N]) {
#pragma unroll
  for (int m = LPE; m < 64; m <<= 1)
#pragma unroll
    for (int t = 0; t < N; ++t) v[t] += __shfl_xor(v[t], m, 64);
}

// Adds the partial sums of waves 1..NW-1 (held by the lanes of edge slot 0)
// to those of wave 0, in wave order, through LDS; every thread of the
// workgroup calls it.
template <int NW, int LPE, int N>
__device__ __forceinline__ void add_wave_partials(float (&acc)[N], float (&red)[NW > 1 ? NW - 1 : 1][LPE][N],
                                                  int wv, int slot, int uu) {
  if constexpr (NW > 1) {
    if (wv > 0 && slot == 0) {
#pragma unroll
      for (int t = 0; t < N; ++t) red[wv - 1][uu][t] = acc[t];
    }
    __syncthreads();
    if (wv == 0) {
#pragma unroll
      for (int v = 0; v < NW - 1; ++v)
#pragma unroll
        for (int t = 0; t < N; ++t) acc[t] += red[v][uu][t];
    }
  }
}

template <class S, int U>
__device__ __forceinline__ void zero_xrow(float (&v)[LaneMap<U>::CPL][S::XC]) {
#pragma unroll
  for (int cc = 0; cc < LaneMap<U>::CPL; ++cc)
#pragma unroll
    for (int a = 0; a < S::XC; ++a) v[cc][a] = 0.f;
}

// edge_bwd_recv with grad_w accumulated instead of assigned
template <class S>
__device__ __forceinline__ void edge_bwd_recv_acc(const float (&xr)[S::XC], const float (&yr)[S::YC],
                                                  const float (&wr)[S::NP], const float (&gr)[S::OC],
                                                  float (&gw)[S::NP], float (&gy)[S::YC]) {
  float t[S::NP];
  edge_bwd_recv<S>(xr, yr, wr, gr, t, gy);
#pragma unroll
  for (int p = 0; p < S::NP; ++p) gw[p] += t[p];
}

template <class S, int U>
__device__ __forceinline__ void load_wrow(const float* __restrict__ w, int e, int u, float (&wr)[S::NP]) {
#pragma unroll
  for (int p = 0; p < S::NP; ++p) wr[p] = w[((size_t)e * S::NP + p) * U + u];
}

// Whether one walk over a receiver's edges can hold every operand of every
// term at once (one channel per lane, and the dg accumulator, the grad_out
// row, both sender rows, the four edge rows and the dw/dY values of an edge
// within about 160 registers); otherwise the receiver pass walks twice.
template <class S, int U>
constexpr bool dbl_one_walk() {
  return LaneMap<U>::CPL == 1 && 2 * S::OC + 2 * S::XC + 3 * S::YC + 3 * S::NP <= 160;
}

// Waves per node in both passes (one channel per lane): the waves of a node
// take every NW-th step of its edges, which keeps several waves per SIMD in
// flight on graphs of a few thousand nodes and splits a hub's edges; the
// per-wave partial sums are added in wave order through LDS.  Two waves
// (measured with the nodes in launch order: Zipf graph 12.4 against 12.9 ms
// with four, 1,536 atoms 107 against 108 us; four had paid in node order,
// where hubs starting late set the end of the launch).
template <int U>
constexpr int dbl_waves() { return LaneMap<U>::CPL == 1 ? 2 : 1; }

// Receiver pass of the second-order backward: dg per receiver, dY and dw per
// edge.  Where the signature allows it, one walk over the receiver's edges
// reads each edge's rows once and produces all three; otherwise dg comes from
// a first walk and dY, dw from a second, each term's operands loaded just
// before it is computed so that large signatures do not hold every operand of
// every term at once.  Per edge the terms are added in the same order either
// way.
template <class S, int U, int NW>
__global__ void __launch_bounds__(64 * NW)
    k_dbl_recv(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col,
               const float* __restrict__ x, const float* __restrict__ Y, const float* __restrict__ w,
               const float* __restrict__ g, const float* __restrict__ ggx, const float* __restrict__ ggY,
               const float* __restrict__ ggw, float* __restrict__ dY, float* __restrict__ dw,
               float* __restrict__ dg, const int32_t* __restrict__ order) {
  using M = LaneMap<U>;
  const int i = launch_node(order, gridDim.x), lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int slot = lane / M::LPE, uu = lane % M::LPE;
  const int beg = row_ptr[i], end = row_ptr[i + 1];
  if constexpr (dbl_one_walk<S, U>()) {
    __shared__ float red[NW > 1 ? NW - 1 : 1][M::LPE][S::OC];
    const bool want_yw = dY || dw;
    float acc[S::OC], gr[1][S::OC];
#pragma unroll
    for (int o = 0; o < S::OC; ++o) acc[o] = 0.f;
    if (want_yw) load_orow<S, U>(g + (size_t)i * (U * S::OC), uu, gr);
    for (int e0 = beg + wv * M::EPW; e0 < end; e0 += NW * M::EPW) {
      const int e = e0 + slot;
      const bool valid = e < end;
      const int ec = valid ? e : end - 1;
      const int j = col[ec];
      float yr[S::YC], gyr[S::YC], wr[S::NP], gwr[S::NP], xr[1][S::XC], gxr[1][S::XC];
#pragma unroll
      for (int b = 0; b < S::YC; ++b) {
        yr[b] = Y[(size_t)ec * S::YC + b];
        gyr[b] = ggY ? ggY[(size_t)ec * S::YC + b] : 0.f;
      }
      load_wrow<S, U>(w, ec, uu, wr);
      if (ggw) load_wrow<S, U>(ggw, ec, uu, gwr);
      else {
#pragma unroll
        for (int p = 0; p < S::NP; ++p) gwr[p] = 0.f;
      }
      load_xrow<S, U>(x + (size_t)j * (U * S::XC), uu, xr);
      if (ggx) load_xrow<S, U>(ggx + (size_t)j * (U * S::XC), uu, gxr);
      if (dg && valid) {
        if (ggx) edge_fwd<S>(gxr[0], yr, wr, acc);     // out(ggx, Y, w)
        if (ggY) edge_fwd<S>(xr[0], gyr, wr, acc);     // out(x, ggY, w)
        if (ggw) edge_fwd<S>(xr[0], yr, gwr, acc);     // out(x, Y, ggw)
      }
      if (want_yw) {
        float tw[S::NP], dyv[S::YC];
#pragma unroll
        for (int p = 0; p < S::NP; ++p) tw[p] = 0.f;
#pragma unroll
        for (int b = 0; b < S::YC; ++b) dyv[b] = 0.f;
        if (ggx) edge_bwd_recv_acc<S>(gxr[0], yr, wr, gr[0], tw, dyv);     // gw(ggx, Y, g), gY(ggx, w, g)
        if (ggY || ggw) edge_bwd_recv_acc<S>(xr[0], gyr, gwr, gr[0], tw, dyv);  // gw(x, ggY, g), gY(x, ggw, g)
        if (dw && valid) {
#pragma unroll
          for (int p = 0; p < S::NP; ++p) dw[((size_t)e * S::NP + p) * U + uu] = tw[p];
        }
        if (dY) {
          lane_sum_halving<S::YC, M::LPE / 2>(dyv, lane);
          if (valid) {
            const HalvingShare sh = halving_share(S::YC, M::LPE, lane);
#pragma unroll
            for (int r = 0; r < ls_final(S::YC, M::LPE); ++r)
              if (r < sh.len) dY[(size_t)e * S::YC + sh.first + r] = dyv[r];
          }
        }
      }
    }
    if (dg) {
      cross_slot_sum<M::LPE, S::OC>(acc);
      add_wave_partials<NW, M::LPE, S::OC>(acc, red, wv, slot, uu);
      if (wv == 0 && slot == 0) {
        float* row = dg + (size_t)i * (U * S::OC);
        static_for<S::NO>([&](auto K) {
          constexpr OutInfo oi = S::outs.o[K];
          constexpr int d = 2 * oi.l + 1;
          static_for<d>([&](auto C) { row[U * oi.ko + uu * d + C] = acc[oi.ko + C]; });
        });
      }
    }
    return;
  }
  static_assert(NW == 1 || M::CPL == 1, "several waves per receiver only with one channel per lane");
  if (dg) {
    __shared__ float red[NW > 1 ? NW - 1 : 1][M::LPE][S::OC];
    float acc[M::CPL][S::OC];
#pragma unroll
    for (int cc = 0; cc < M::CPL; ++cc)
#pragma unroll
      for (int o = 0; o < S::OC; ++o) acc[cc][o] = 0.f;
    for (int e0 = beg + wv * M::EPW; e0 < end; e0 += NW * M::EPW) {
      const int e = e0 + slot;
      if (e < end) {
        const int j = col[e];
        float yr[S::YC];
#pragma unroll
        for (int b = 0; b < S::YC; ++b) yr[b] = Y[(size_t)e * S::YC + b];
#pragma unroll
        for (int cc = 0; cc < M::CPL; ++cc) {
          const int u = uu + 64 * cc;
          float wr[S::NP], xr[M::CPL][S::XC];
          load_wrow<S, U>(w, e, u, wr);
          if (ggx) {                                   // out(ggx, Y, w)
            load_xrow<S, U>(ggx + (size_t)j * (U * S::XC), uu, xr);
            edge_fwd<S>(xr[cc], yr, wr, acc[cc]);
            __builtin_amdgcn_sched_barrier(0);
          }
          load_xrow<S, U>(x + (size_t)j * (U * S::XC), uu, xr);
          if (ggY) {                                   // out(x, ggY, w)
            float gyr[S::YC];
#pragma unroll
            for (int b = 0; b < S::YC; ++b) gyr[b] = ggY[(size_t)e * S::YC + b];
            edge_fwd<S>(xr[cc], gyr, wr, acc[cc]);
            __builtin_amdgcn_sched_barrier(0);
          }
          if (ggw) {                                   // out(x, Y, ggw)
            load_wrow<S, U>(ggw, e, u, wr);
            edge_fwd<S>(xr[cc], yr, wr, acc[cc]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
#pragma unroll
    for (int cc = 0; cc < M::CPL; ++cc) cross_slot_sum<M::LPE, S::OC>(acc[cc]);
    add_wave_partials<NW, M::LPE, S::OC>(acc[0], red, wv, slot, uu);
    if (wv == 0 && slot == 0) {
      float* row = dg + (size_t)i * (U * S::OC);
      static_for<S::NO>([&](auto K) {
        constexpr OutInfo oi = S::outs.o[K];
        constexpr int d = 2 * oi.l + 1;
#pragma unroll
        for (int cc = 0; cc < M::CPL; ++cc)
          static_for<d>([&](auto C) { row[U * oi.ko + (uu + 64 * cc) * d + C] = acc[cc][oi.ko + C]; });
      });
    }
  }
  if (dY || dw) {
    float gr[M::CPL][S::OC];
    load_orow<S, U>(g + (size_t)i * (U * S::OC), uu, gr);
    for (int e0 = beg + wv * M::EPW; e0 < end; e0 += NW * M::EPW) {
      const int e = e0 + slot;
      const bool valid = e < end;
      const int ec = valid ? e : end - 1;
      const int j = col[ec];
      float dyv[S::YC];
#pragma unroll
      for (int b = 0; b < S::YC; ++b) dyv[b] = 0.f;
#pragma unroll
      for (int cc = 0; cc < M::CPL; ++cc) {
        const int u = uu + 64 * cc;
        float tw[S::NP];
#pragma unroll
        for (int p = 0; p < S::NP; ++p) tw[p] = 0.f;
        if (ggx) {                                     // gw(ggx, Y, g), gY(ggx, w, g)
          float xr[M::CPL][S::XC], yr[S::YC], wr[S::NP];
          load_xrow<S, U>(ggx + (size_t)j * (U * S::XC), uu, xr);
#pragma unroll
          for (int b = 0; b < S::YC; ++b) yr[b] = Y[(size_t)ec * S::YC + b];
          load_wrow<S, U>(w, ec, u, wr);
          edge_bwd_recv_acc<S>(xr[cc], yr, wr, gr[cc], tw, dyv);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (ggY || ggw) {                              // gw(x, ggY, g), gY(x, ggw, g)
          float xr[M::CPL][S::XC], yr[S::YC], wr[S::NP];
          load_xrow<S, U>(x + (size_t)j * (U * S::XC), uu, xr);
#pragma unroll
          for (int b = 0; b < S::YC; ++b) yr[b] = ggY ? ggY[(size_t)ec * S::YC + b] : 0.f;
          if (ggw) load_wrow<S, U>(ggw, ec, u, wr);
          else {
#pragma unroll
            for (int p = 0; p < S::NP; ++p) wr[p] = 0.f;
          }
          edge_bwd_recv_acc<S>(xr[cc], yr, wr, gr[cc], tw, dyv);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (dw && valid) {
#pragma unroll
          for (int p = 0; p < S::NP; ++p) dw[((size_t)e * S::NP + p) * U + u] = tw[p];
        }
      }
      if (dY) {
        lane_sum_halving<S::YC, M::LPE / 2>(dyv, lane);
        if (valid) {
          const HalvingShare sh = halving_share(S::YC, M::LPE, lane);
#pragma unroll
          for (int r = 0; r < ls_final(S::YC, M::LPE); ++r)
            if (r < sh.len) dY[(size_t)e * S::YC + sh.first + r] = dyv[r];
        }
      }
    }
  }
}

template <class S, int U, int NW>
__global__ void __launch_bounds__(64 * NW)
    k_dbl_send(const int32_t* __restrict__ t_row_ptr, const int32_t* __restrict__ t_perm,
               const int32_t* __restrict__ t_col, const float* __restrict__ Y, const float* __restrict__ w,
               const float* __restrict__ g, const float* __restrict__ ggY, const float* __restrict__ ggw,
               float* __restrict__ dx, const int32_t* __restrict__ order) {
  using M = LaneMap<U>;
  const int j = launch_node(order, gridDim.x), lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int slot = lane / M::LPE, uu = lane % M::LPE;
  const int beg = t_row_ptr[j], end = t_row_ptr[j + 1];
  float acc[M::CPL][S::XC];
  zero_xrow<S, U>(acc);
  for (int e0 = beg + wv * M::EPW; e0 < end; e0 += NW * M::EPW) {
    const int t = e0 + slot;
    if (t < end) {
      const int e = t_perm[t], i = t_col[t];
      float yr[S::YC], gyr[S::YC];
#pragma unroll
      for (int b = 0; b < S::YC; ++b) {
        yr[b] = Y[(size_t)e * S::YC + b];
        gyr[b] = ggY ? ggY[(size_t)e * S::YC + b] : 0.f;
      }
      float gr[M::CPL][S::OC];
      load_orow<S, U>(g + (size_t)i * (U * S::OC), uu, gr);
#pragma unroll
      for (int cc = 0; cc < M::CPL; ++cc) {
        const int u = uu + 64 * cc;
        float wr[S::NP], gwr[S::NP];
#pragma unroll
        for (int p = 0; p < S::NP; ++p) {
          wr[p] = w[((size_t)e * S::NP + p) * U + u];
          gwr[p] = ggw ? ggw[((size_t)e * S::NP + p) * U + u] : 0.f;
        }
        edge_bwd_send<S>(gyr, wr, gr[cc], acc[cc]);
        edge_bwd_send<S>(yr, gwr, gr[cc], acc[cc]);
      }
    }
  }
#pragma unroll
  for (int cc = 0; cc < M::CPL; ++cc) cross_slot_sum<M::LPE, S::XC>(acc[cc]);
  static_assert(NW == 1 || M::CPL == 1, "several waves per sender only with one channel per lane");
  __shared__ float red[NW > 1 ? NW - 1 : 1][M::LPE][S::XC];
  add_wave_partials<NW, M::LPE, S::XC>(acc[0], red, wv, slot, uu);
  if (wv == 0 && slot == 0) {
    float* row = dx + (size_t)j * (U * S::XC);
    static_for<S::NIN>([&](auto I) {
      constexpr int d = 2 * S::ls.v[I] + 1;
      constexpr int xo = S::xoff(I);
#pragma unroll
      for (int cc = 0; cc < M::CPL; ++cc)
        static_for<d>([&](auto A) { row[U * xo + (uu + 64 * cc) * d + A] = acc[cc][xo + A]; });
    });
  }
}

template <class S, int U>
hipError_t launch_dbl_recv(const ConvArgs& a) {
  if (a.n_nodes == 0 || (!a.d_Y && !a.d_w && !a.d_g)) return hipSuccess;
  constexpr int NW = dbl_waves<U>();
  hipLaunchKernelGGL((k_dbl_recv<S, U, NW>), dim3(a.n_nodes), dim3(64 * NW), 0, a.stream, a.row_ptr, a.col, a.x, a.Y,
                     a.w, a.grad_out, a.gg_x, a.gg_Y, a.gg_w, a.d_Y, a.d_w, a.d_g, a.r_order);
  return hipGetLastError();
}

template <class S, int U>
hipError_t launch_dbl_send(const ConvArgs& a) {
  if (a.n_nodes == 0 || !a.d_x) return hipSuccess;
  constexpr int NW = dbl_waves<U>();
  hipLaunchKernelGGL((k_dbl_send<S, U, NW>), dim3(a.n_nodes), dim3(64 * NW), 0, a.stream, a.t_row_ptr, a.t_perm,
                     a.t_col, a.Y, a.w, a.grad_out, a.gg_Y, a.gg_w, a.d_x, a.s_order);
  return hipGetLastError();
}

}  // namespace tpc
