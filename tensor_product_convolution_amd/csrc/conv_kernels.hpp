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
//   * one pass (lmax-2 signatures, every gradient requested): each workgroup
//     owns a sender j with x[j] in registers, walks its edges in the sender
//     grouping, gathers grad_out of each receiver, writes grad_w[e] and
//     grad_Y[e] at the edge's receiver-sorted position and stores grad_x[j]
//     once, so w and Y are read once per backward;
//   * otherwise a receiver pass: with grad_out[i] in registers, each edge
//     yields grad_w[e] (per lane) and grad_Y[e] (a recursive-halving sum over
//     the edge's channel lanes), written once per edge -- these are
//     requested outputs;
//   * and a sender pass: each workgroup owns a sender j and walks its edges
//     in the sender grouping, gathering grad_out of each receiver, and stores
//     grad_x[j] once.  No atomics anywhere.
#pragma once
#include "internal.hpp"
#include "sh_eval.hpp"
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

// Sums of N values over the lanes that differ in the bits below 2 OFF (for
// example the channel lanes of one edge), by recursive halving: at the stage
// with lane offset OFF a lane keeps one half of its list (the upper half if
// its OFF bit is set), sends the other half to the partner lane and adds what
// the partner sent, so a stage costs ceil(N / 2) exchanges instead of N.
// After the last stage a lane holds ls_final(N, 2 OFF) totals, the first of
// which is value sum over stages of (bit ? ceil(n / 2) : 0), n the list
// length at that stage; slots past the real values hold zeros.
constexpr int ls_final(int n, int lanes) { return lanes <= 1 ? n : ls_final((n + 1) / 2, lanes / 2); }

template <int N, int OFF, int CAP>
__device__ __forceinline__ void lane_sum_halving(float (&v)[CAP], int lane) {
  if constexpr (OFF >= 1) {
    constexpr int H = (N + 1) / 2;
    const bool bit = (lane & OFF) != 0;
#pragma unroll
    for (int q = 0; q < H; ++q) {
      const float lo = v[q], hi = q + H < N ? v[q + H] : 0.f;
      const float keep = bit ? hi : lo, send = bit ? lo : hi;
      v[q] = keep + __shfl_xor(send, OFF, 64);
    }
    lane_sum_halving<H, OFF / 2>(v, lane);
  }
}

// the values a lane holds after lane_sum_halving over LANES lanes of a list of N
struct HalvingShare {
  int first, len;
};
__device__ __forceinline__ HalvingShare halving_share(int n, int lanes, int lane) {
  HalvingShare s{0, n};
  for (int off = lanes / 2; off >= 1; off >>= 1) {
    const int h = (n + 1) / 2;
    if (lane & off) {
      s.first += h;
      s.len = s.len > h ? s.len - h : 0;
    } else {
      s.len = s.len < h ? s.len : h;
    }
    n = h;
  }
  return s;
}

// ---------------------------------------------------------------------------
// per-edge arithmetic of one channel
//
// For large signatures the arithmetic is cut into phases at every change of
// (input irrep, l2): the accumulators and the inputs pass through an empty asm
// statement there, so every product of one group is formed after the previous
// group has been folded into the accumulators.  Without it the code generator
// forms the partial sums of all paths first (the instruction-selection DAG
// orders pure arithmetic freely) and holds hundreds of them live, which cuts
// occupancy to one wave per SIMD and adds register spills.  Small signatures
// are left to the scheduler.

template <class S>
constexpr bool kPhased = S::nnz_total() > 256;

template <class S, int P>
constexpr bool group_end() {
  if constexpr (P + 1 < S::NP) {
    constexpr PathInfo a = S::paths.p[P], b = S::paths.p[P + 1];
    return a.in != b.in || a.l2 != b.l2;
  }
  return false;
}

template <int N>
__device__ __forceinline__ void launder(float (&v)[N]) {
#pragma unroll
  for (int t = 0; t < N; ++t) asm volatile("" : "+v"(v[t]));
}

// out accumulators += sum_p w_p * sum_nz C x_a Y_b
template <class S>
__device__ __forceinline__ void edge_fwd(const float (&xin)[S::XC], const float (&yin)[S::YC],
                                         const float (&wr)[S::NP], float (&acc)[S::OC]) {
  float xr[S::XC], yr[S::YC];
#pragma unroll
  for (int a = 0; a < S::XC; ++a) xr[a] = xin[a];
#pragma unroll
  for (int b = 0; b < S::YC; ++b) yr[b] = yin[b];
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
    if constexpr (kPhased<S> && group_end<S, P>()) {
      launder(acc);
      launder(xr);
      launder(yr);
    }
  });
}

// Z_p[b] = sum_{a,c} C x_a g_c ; grad_w_p = sum_b Y_b Z_p[b] ; grad_Y_b += w_p Z_p[b]
// (the products x_a g_c are shared by every path with the same (l1, output irrep))
template <class S>
__device__ __forceinline__ void edge_bwd_recv(const float (&xin)[S::XC], const float (&yr)[S::YC],
                                              const float (&wr)[S::NP], const float (&gin)[S::OC],
                                              float (&gw)[S::NP], float (&gy)[S::YC]) {
  float xr[S::XC], gr[S::OC];
#pragma unroll
  for (int a = 0; a < S::XC; ++a) xr[a] = xin[a];
#pragma unroll
  for (int c = 0; c < S::OC; ++c) gr[c] = gin[c];
  static_for<S::NP>([&](auto P) {
    constexpr PathInfo pi = S::paths.p[P];
    using T = CgPath<pi.l1, pi.l2, pi.l3>;
    constexpr int D2 = 2 * pi.l2 + 1;
    float z[D2];
    static_for<D2>([&](auto B) { z[B] = 0.f; });
    static_for<T::nnz>([&](auto N) {
      constexpr Nz e = T::table.e[N];
      z[e.b] = fmaf(e.v, xr[pi.xo + e.a] * gr[pi.ko + e.c], z[e.b]);
    });
    float s = 0.f;
    static_for<D2>([&](auto B) { s = fmaf(yr[pi.yo + B], z[B], s); });
    gw[P] = s;
    static_for<D2>([&](auto B) { gy[pi.yo + B] = fmaf(wr[P], z[B], gy[pi.yo + B]); });
    if constexpr (kPhased<S> && group_end<S, P>()) {
      launder(gy);
      launder(gw);
      launder(xr);
      launder(gr);
    }
  });
}

// grad_x_a += sum_p w_p sum_nz C Y_b g_c, grouped by (input irrep, l2): the
// paths of a group share the x block and the Y block, so
//   V[a][b] = sum_{p in group} w_p sum_c C_p[a,b,c] g[c]
// is formed first and folded with Y once per group, grad_x_a += sum_b Y_b
// V[a][b] (the adjoint of the forward's shared products x_a Y_b): per edge and
// channel nnz + sum_p (2l3+1) + the coupled (a, b) pairs of each group
// (1,023 operations at lmax 3) instead of 2 nnz + sum_p (2l3+1) (1,378).
template <class S, int P>
constexpr bool group_first() {
  if constexpr (P > 0) {
    constexpr PathInfo a = S::paths.p[P - 1], b = S::paths.p[P];
    return a.in != b.in || a.l2 != b.l2;
  }
  return true;
}

// does some path of the group (l1, l2, l3 = |l1-l2| .. min(l1+l2, lout))
// couple x component a with Y component b?
constexpr bool group_couples(int l1, int l2, int lout, int a, int b) {
  const int lo = l1 > l2 ? l1 - l2 : l2 - l1, hi = l1 + l2 < lout ? l1 + l2 : lout;
  for (int l3 = lo; l3 <= hi; ++l3)
    for (int c = 0; c <= 2 * l3; ++c) {
      const double v = real_cg_raw(l1, l2, l3, a, b, c);
      if (v > kZeroTol || v < -kZeroTol) return true;
    }
  return false;
}

template <class S>
__device__ __forceinline__ void edge_bwd_send(const float (&yin)[S::YC], const float (&wr)[S::NP],
                                              const float (&gin)[S::OC], float (&gx)[S::XC]) {
  float yr[S::YC], gr[S::OC];
#pragma unroll
  for (int b = 0; b < S::YC; ++b) yr[b] = yin[b];
#pragma unroll
  for (int c = 0; c < S::OC; ++c) gr[c] = gin[c];
  float V[7 * 7];   // one group's (2l1+1) x (2l2+1), l <= 3
  static_for<S::NP>([&](auto P) {
    constexpr PathInfo pi = S::paths.p[P];
    using T = CgPath<pi.l1, pi.l2, pi.l3>;
    constexpr int D1 = 2 * pi.l1 + 1, D2 = 2 * pi.l2 + 1, D3 = 2 * pi.l3 + 1;
    static_assert(D1 * D2 <= 7 * 7, "degrees up to 3");
    if constexpr (group_first<S, P>()) static_for<D1 * D2>([&](auto I) { V[I] = 0.f; });
    float wg[D3];
    static_for<D3>([&](auto C) { wg[C] = wr[P] * gr[pi.ko + C]; });
    static_for<T::nnz>([&](auto N) {
      constexpr Nz z = T::table.e[N];
      V[z.a * D2 + z.b] = fmaf(z.v, wg[z.c], V[z.a * D2 + z.b]);
    });
    if constexpr (P + 1 == S::NP || group_end<S, P>()) {
      static_for<D1>([&](auto A) {
        static_for<D2>([&](auto B) {
          if constexpr (group_couples(pi.l1, pi.l2, S::lmax_out, A, B))
            gx[pi.xo + A] = fmaf(yr[pi.yo + B], V[A * D2 + B], gx[pi.xo + A]);
        });
      });
      if constexpr (kPhased<S>) {
        launder(gx);
        launder(yr);
        launder(gr);
      }
    }
  });
}

// ---------------------------------------------------------------------------
// All three backward terms of one edge and channel in one pass.
//
// Every CG nonzero C_p[a,b,c] of a path that lands on output component
// o = ko(p) + c meets the upstream gradient only as the product C g_o, and its
// magnitude |C| takes few distinct values per component.  So the distinct
// scaled values gC = |C| g_o (|C| != 1) are formed once per edge and channel
// and shared by every path on that output irrep; each nonzero is then one
// fused multiply-add with a sign modifier for each of the two contractions:
//   Z_p[b]  += sign(C) x_a gC     (grad_w_p = sum_b Y_b Z_p[b];
//                                  grad_Y_b += w_p Z_p[b])
//   V[a][b] += sign(C) w_p gC     (per (input irrep, l2) group;
//                                  grad_x_a += sum_b Y_b V[a][b])
// On the lmax-2 signature of three inputs this is 42 scalings + 2 x 137
// nonzero FMAs + 102 + 81 folds, against 645 operations for the receiver-side
// Z form and the sender-side grouped adjoint evaluated separately.
template <class S>
struct ScaledG {
  struct Ent {
    int o;
    float v;
  };
  struct Table {
    Ent e[512];
    int n;
  };
  static constexpr Table build() {
    Table t{};
    t.n = 0;
    for (int p = 0; p < S::NP; ++p) {
      const PathInfo pi = S::paths.p[p];
      const double sg = real_cg_sign(pi.l1, pi.l2, pi.l3);
      for (int a = 0; a <= 2 * pi.l1; ++a)
        for (int b = 0; b <= 2 * pi.l2; ++b)
          for (int c = 0; c <= 2 * pi.l3; ++c) {
            const float v = static_cast<float>(real_cg(pi.l1, pi.l2, pi.l3, a, b, c, sg));
            const float m = v < 0.f ? -v : v;
            if (m == 0.f || m == 1.f) continue;
            const int o = pi.ko + c;
            bool seen = false;
            for (int q = 0; q < t.n; ++q)
              if (t.e[q].o == o && t.e[q].v == m) seen = true;
            if (!seen) t.e[t.n++] = Ent{o, m};
          }
    }
    return t;
  }
  static constexpr Table table = build();
  static constexpr int N = table.n;
  static_assert(N <= 512, "scaled-gradient table");
  // slot of (component o, magnitude m) in the table; -1 for m == 1
  static constexpr int find(int o, float m) {
    for (int q = 0; q < N; ++q)
      if (table.e[q].o == o && table.e[q].v == m) return q;
    return -1;
  }
};

// ym: Y for the sender-side fold (zero on a slot whose grad_x share is
// dropped); gw is assigned, gy and gx accumulate.
template <class S>
__host__ __device__ __forceinline__ void edge_bwd_all(const float (&xin)[S::XC], const float (&yr)[S::YC],
                                                      const float (&ym)[S::YC], const float (&wr)[S::NP],
                                                      const float (&gin)[S::OC], float (&gw)[S::NP],
                                                      float (&gy)[S::YC], float (&gx)[S::XC]) {
  using G = ScaledG<S>;
  float xr[S::XC], gr[S::OC];
#pragma unroll
  for (int a = 0; a < S::XC; ++a) xr[a] = xin[a];
#pragma unroll
  for (int c = 0; c < S::OC; ++c) gr[c] = gin[c];
  float gc[G::N > 0 ? G::N : 1];
  static_for<G::N>([&](auto I) { gc[I] = G::table.e[I].v * gr[G::table.e[I].o]; });
  float V[7 * 7];   // one group's (2l1+1) x (2l2+1), l <= 3
  static_for<S::NP>([&](auto P) {
    constexpr PathInfo pi = S::paths.p[P];
    using T = CgPath<pi.l1, pi.l2, pi.l3>;
    constexpr int D1 = 2 * pi.l1 + 1, D2 = 2 * pi.l2 + 1;
    static_assert(D1 * D2 <= 7 * 7, "degrees up to 3");
    if constexpr (group_first<S, P>()) static_for<D1 * D2>([&](auto I) { V[I] = 0.f; });
    float z[D2];
    static_for<D2>([&](auto B) { z[B] = 0.f; });
    static_for<T::nnz>([&](auto Nn) {
      constexpr Nz e = T::table.e[Nn];
      constexpr int o = pi.ko + e.c;
      constexpr float m = e.v < 0.f ? -e.v : e.v;
      constexpr int gi = m == 1.f ? -1 : G::find(o, m);
      static_assert(m == 1.f || gi >= 0, "scaled-gradient slot");
      const float gv = gi >= 0 ? gc[gi >= 0 ? gi : 0] : gr[o];
      const float xs = e.v < 0.f ? -xr[pi.xo + e.a] : xr[pi.xo + e.a];
      const float ws = e.v < 0.f ? -wr[P] : wr[P];
      z[e.b] = fmaf(xs, gv, z[e.b]);
      V[e.a * D2 + e.b] = fmaf(ws, gv, V[e.a * D2 + e.b]);
    });
    float sw = 0.f;
    static_for<D2>([&](auto B) { sw = fmaf(yr[pi.yo + B], z[B], sw); });
    gw[P] = sw;
    static_for<D2>([&](auto B) { gy[pi.yo + B] = fmaf(wr[P], z[B], gy[pi.yo + B]); });
    if constexpr (P + 1 == S::NP || group_end<S, P>()) {
      static_for<D1>([&](auto A) {
        static_for<D2>([&](auto B) {
          if constexpr (group_couples(pi.l1, pi.l2, S::lmax_out, A, B))
            gx[pi.xo + A] = fmaf(ym[pi.yo + B], V[A * D2 + B], gx[pi.xo + A]);
        });
      });
      if constexpr (kPhased<S>) {
        launder(gx);
        launder(gy);
        launder(gw);
        launder(xr);
        launder(gr);
      }
    }
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
// LDS staging of edge operands
//
// Each wave streams its edges through a private double buffer in LDS filled by
// gfx950's direct global->LDS loads (global_load_lds_dwordx4: every lane moves
// 16 bytes, one instruction moves 1 KB, no VGPRs involved).  While the wave
// computes step k from buffer k&1, the loads of step k+1 fill the other
// buffer; a wait on the vector-memory counter with the number of loads just
// issued ensures step k's data has landed.  The edges of one wave step are
// consecutive in the receiver-sorted order, so their weight and Y rows are one
// contiguous run; x (or grad_out) rows are gathered row by row.  Indices past
// the segment are clamped to its last edge so every load is in bounds.

typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void gbl_void_t;

// s_waitcnt vmcnt(n) (expcnt / lgkmcnt left at their maxima), n < 64
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

constexpr int ceil16(int bytes) { return (bytes + 15) / 16 * 16; }

// Copy NR rows of RB bytes (RB % 16 == 0) to LDS at dst, rows back to back.
// row(r) returns the global address of row r.  Issues ceil(NR*RB/1024) loads.
// cache policy of a staging load: streams read once are non-temporal so they do
// not evict data that is re-read (x rows, grad_out rows) from L2
constexpr int kTemporal = 0;
constexpr int kStream = 2;   // nt

template <int NR, int RB, int POL = kTemporal, class RowFn>
__device__ __forceinline__ void dma_rows16(char* dst, RowFn row, int lane) {
  static_assert(RB % 16 == 0, "row bytes must be a multiple of 16");
  constexpr int CH = RB / 16, N = NR * CH, INSTR = (N + 63) / 64;
  static_for<INSTR>([&](auto K) {
    const int c = K * 64 + lane;
    if (K * 64 + 64 <= N || c < N) {
      const int r = c / CH;
      const char* src = row(r) + (c - r * CH) * 16;
      __builtin_amdgcn_global_load_lds((gbl_void_t*)src, (lds_void_t*)(dst + K * 1024), 16, 0, POL);
    }
  });
}
template <int NR, int RB>
constexpr int dma16_count() { return (NR * (RB / 16) + 63) / 64; }

// Same with 4-byte granules (rows of any multiple of 4 bytes).
template <int NR, int RB, int POL = kTemporal, class RowFn>
__device__ __forceinline__ void dma_rows4(char* dst, RowFn row, int lane) {
  static_assert(RB % 4 == 0, "row bytes must be a multiple of 4");
  constexpr int CH = RB / 4, N = NR * CH, INSTR = (N + 63) / 64;
  static_for<INSTR>([&](auto K) {
    const int c = K * 64 + lane;
    if (K * 64 + 64 <= N || c < N) {
      const int r = c / CH;
      const char* src = row(r) + (c - r * CH) * 4;
      __builtin_amdgcn_global_load_lds((gbl_void_t*)src, (lds_void_t*)(dst + K * 256), 4, 0, POL);
    }
  });
}
template <int NR, int RB>
constexpr int dma4_count() { return (NR * (RB / 4) + 63) / 64; }

// select v[r] from a small wave-uniform array with a constant-index chain
template <int N>
__device__ __forceinline__ int pick(const int (&v)[N], int r) {
  int o = v[0];
#pragma unroll
  for (int t = 1; t < N; ++t) o = r == t ? v[t] : o;
  return o;
}

// Per-wave staging layout for receiver-grouped passes: [W | Y | X] per buffer.
// GEOM: the edge rows staged are the edge vectors r (3 floats) instead of Y,
// and the harmonics are evaluated on chip (read_y).
template <class S, int U, bool GEOM = false>
struct RecvStage {
  static constexpr int EPW = LaneMap<U>::EPW;
  static constexpr int WB = S::NP * U * 4;       // weight row bytes
  static constexpr int YR = GEOM ? 3 : S::YC;    // floats of an edge's geometry row
  static constexpr int YB = YR * 4;              // Y (or r) row bytes
  static constexpr int XB = S::XC * U * 4;       // x row bytes
  static constexpr int W_OFF = 0;
  static constexpr int Y_OFF = ceil16(EPW * WB);
  static constexpr int X_OFF = Y_OFF + ceil16(EPW * YB);
  static constexpr int BUF = X_OFF + EPW * XB;   // bytes per buffer
  static constexpr int NLOADS = dma16_count<EPW, WB>() + dma4_count<EPW, YB>() + dma16_count<EPW, XB>();
};

// issue the loads of the wave step starting at segment position q0
template <class S, int U, bool GEOM = false>
__device__ __forceinline__ void stage_recv(char* buf, const float* __restrict__ x,
                                           const float* __restrict__ Y, const float* __restrict__ w,
                                           const int (&j)[LaneMap<U>::EPW], int q0, int last,
                                           int lane) {
  using T = RecvStage<S, U, GEOM>;
  dma_rows16<T::EPW, T::WB, kStream>(buf + T::W_OFF, [&](int r) {
    return (const char*)(w + (size_t)min(q0 + r, last) * (S::NP * U));
  }, lane);
  dma_rows4<T::EPW, T::YB, kStream>(buf + T::Y_OFF, [&](int r) {
    return (const char*)(Y + (size_t)min(q0 + r, last) * T::YR);
  }, lane);
  dma_rows16<T::EPW, T::XB>(buf + T::X_OFF, [&](int r) {
    return (const char*)(x + (size_t)pick(j, r) * (S::XC * U));
  }, lane);
}

// the same step when the edge rows are stored in the sender grouping: the
// weight and Y rows of the step's edges are gathered at rows e[r]
template <class S, int U, bool GEOM = false>
__device__ __forceinline__ void stage_recv_at(char* buf, const float* __restrict__ x,
                                              const float* __restrict__ Y, const float* __restrict__ w,
                                              const int (&j)[LaneMap<U>::EPW],
                                              const int (&e)[LaneMap<U>::EPW], int lane) {
  using T = RecvStage<S, U, GEOM>;
  dma_rows16<T::EPW, T::WB, kStream>(buf + T::W_OFF, [&](int r) {
    return (const char*)(w + (size_t)pick(e, r) * (S::NP * U));
  }, lane);
  dma_rows4<T::EPW, T::YB, kStream>(buf + T::Y_OFF, [&](int r) {
    return (const char*)(Y + (size_t)pick(e, r) * T::YR);
  }, lane);
  dma_rows16<T::EPW, T::XB>(buf + T::X_OFF, [&](int r) {
    return (const char*)(x + (size_t)pick(j, r) * (S::XC * U));
  }, lane);
}

// the edge's harmonics from its staged row: Y itself or, with GEOM, evaluated
// from the staged edge vector (the unit direction and 1/|r| go to geo for the
// backward's pullback to r)
template <class S, bool GEOM>
__device__ __forceinline__ void read_y(const float* Yv, float (&yr)[S::YC], float (&geo)[4]) {
  if constexpr (GEOM) {
    float x = Yv[0], y = Yv[1], z = Yv[2], inv;
    unit_dir(x, y, z, inv);
    sh_eval<S::lmax_sh>(x, y, z, yr);
    geo[0] = x;
    geo[1] = y;
    geo[2] = z;
    geo[3] = inv;
  } else {
#pragma unroll
    for (int b = 0; b < S::YC; ++b) yr[b] = Yv[b];
  }
}

// This lane's share of an edge's gradient after the sum over the edge's
// channel lanes: grad_Y or, with GEOM, grad_r, the pullback of grad_Y to the
// edge vector (linear, so the per-lane partials are pulled back first and 3
// values summed instead of (lmax+1)^2).
template <class S, bool GEOM, int LPE, int NOUT>
__device__ __forceinline__ void edge_grad_share(float (&gy)[S::YC], const float (&geo)[4], int lane,
                                                float (&out)[NOUT]) {
  if constexpr (GEOM) {
    float g3[3];
    sh_pullback<S::lmax_sh>(geo[0], geo[1], geo[2], geo[3], gy, 0.f, g3);
    lane_sum_halving<3, LPE / 2>(g3, lane);
#pragma unroll
    for (int r = 0; r < NOUT; ++r) out[r] = g3[r];
  } else {
    lane_sum_halving<S::YC, LPE / 2>(gy, lane);
#pragma unroll
    for (int r = 0; r < NOUT; ++r) out[r] = gy[r];
  }
}

// read this lane's operands of its edge slot from a staged buffer
template <class S, int U, bool GEOM = false>
__device__ __forceinline__ void read_recv(const char* buf, int slot, int uu,
                                          float (&xr)[LaneMap<U>::CPL][S::XC], float (&yr)[S::YC],
                                          float (&wr)[LaneMap<U>::CPL][S::NP], float (&geo)[4]) {
  using T = RecvStage<S, U, GEOM>;
  const float* W = (const float*)(buf + T::W_OFF) + slot * (S::NP * U);
  const float* Yv = (const float*)(buf + T::Y_OFF) + slot * T::YR;
  const float* X = (const float*)(buf + T::X_OFF) + slot * (S::XC * U);
  read_y<S, GEOM>(Yv, yr, geo);
#pragma unroll
  for (int p = 0; p < S::NP; ++p)
#pragma unroll
    for (int cc = 0; cc < LaneMap<U>::CPL; ++cc) wr[cc][p] = W[p * U + uu + 64 * cc];
  static_for<S::NIN>([&](auto I) {
    constexpr int d = 2 * S::ls.v[I] + 1;
    constexpr int xo = S::xoff(I);
#pragma unroll
    for (int cc = 0; cc < LaneMap<U>::CPL; ++cc) {
      const float* p = X + U * xo + (uu + 64 * cc) * d;
      static_for<d>([&](auto A) { xr[cc][xo + A] = p[A]; });
    }
  });
}

// sender-grouped pass: [W | Y | G] per buffer, all rows gathered
template <class S, int U, bool GEOM = false>
struct SendStage {
  static constexpr int EPW = LaneMap<U>::EPW;
  static constexpr int WB = S::NP * U * 4;
  static constexpr int YR = GEOM ? 3 : S::YC;
  static constexpr int YB = YR * 4;
  static constexpr int GB = S::OC * U * 4;
  static constexpr int W_OFF = 0;
  static constexpr int Y_OFF = ceil16(EPW * WB);
  static constexpr int G_OFF = Y_OFF + ceil16(EPW * YB);
  static constexpr int BUF = G_OFF + EPW * GB;
  static constexpr int NLOADS = dma16_count<EPW, WB>() + dma4_count<EPW, YB>() + dma16_count<EPW, GB>();
};

template <class S, int U, bool GEOM = false>
__device__ __forceinline__ void stage_send(char* buf, const float* __restrict__ Y,
                                           const float* __restrict__ w, const float* __restrict__ g,
                                           const int (&q)[LaneMap<U>::EPW],
                                           const int (&i)[LaneMap<U>::EPW], int lane) {
  using T = SendStage<S, U, GEOM>;
  dma_rows16<T::EPW, T::WB, kStream>(buf + T::W_OFF, [&](int r) {
    return (const char*)(w + (size_t)pick(q, r) * (S::NP * U));
  }, lane);
  dma_rows4<T::EPW, T::YB, kStream>(buf + T::Y_OFF, [&](int r) {
    return (const char*)(Y + (size_t)pick(q, r) * T::YR);
  }, lane);
  dma_rows16<T::EPW, T::GB>(buf + T::G_OFF, [&](int r) {
    return (const char*)(g + (size_t)pick(i, r) * (S::OC * U));
  }, lane);
}

// Node of this workgroup: the grid walks the nodes in the given launch order
// (largest degree first, so the longest workgroups do not start last), or in
// node order without one.  Entries are clamped into [0, n).
__device__ __forceinline__ int launch_node(const int32_t* __restrict__ order, int n) {
  const int b = blockIdx.x;
  return order ? min(max(order[b], 0), n - 1) : b;
}

// ---------------------------------------------------------------------------
// kernels
//
// Slot s of wave v owns segment positions beg + v*EPW + s + k*SLOTS.  Every
// wave runs the trip count of its first slot; a slot past the segment works on
// the clamped last edge and its contribution is masked (forward, sender pass)
// or it rewrites exactly the values of that edge (receiver pass).
//
// Pipeline: NBUF staging buffers per wave; step k is computed from buffer
// k % NBUF while the loads of steps k+1 .. k+NBUF-1 are in flight.  Before
// computing step k the wave waits until at most "ops issued after step k's
// loads" vector-memory operations are outstanding; that count is exact
// (DMA loads per step, plus the receiver pass's per-step stores), so the wait
// never drains the loads of later steps.

template <int U, int WPB>
__device__ __forceinline__ int wave_trips(int beg, int end, int wv) {
  using M = LaneMap<U>;
  constexpr int SLOTS = WPB * M::EPW;
  const int first = beg + wv * M::EPW;
  const int n = first < end ? (end - first + SLOTS - 1) / SLOTS : 0;
  return __builtin_amdgcn_readfirstlane(n);
}

// Per-wave window of an int32 index array (col, t_perm, t_col): lane t holds
// the entry of the wave's position for step kbase + t / EPW, slot t % EPW
// (clamped to the segment's last edge), so a step's indices are register
// reads (v_readlane) instead of scalar loads.  A scalar load issued inside the
// step loop shares its counter with the LDS reads, and the wait for those
// would stall on every index line the scalar cache misses.  A window covers
// 64 / EPW steps; longer walks reload it (a vector load, waited for once).
template <int EPW, int SLOTS>
struct IdxWindow {
  static constexpr int STEPS = 64 / EPW;
  int v = 0;
  int kbase = 0;
  __device__ __forceinline__ void load(const int32_t* __restrict__ a, int k00, int kb, int last, int lane) {
    kbase = kb;
    v = a[min(k00 + (kb + lane / EPW) * SLOTS + lane % EPW, last)];
  }
  // entry of slot r at wave step k; reloads first if k is past the window.
  // The reload waits for itself on its own path, so that no load of v is
  // pending where the paths meet (otherwise the code generator would wait
  // for every vector-memory operation before each read of the window).
  __device__ __forceinline__ int get(const int32_t* __restrict__ a, int k00, int k, int r, int last, int lane) {
    if (k - kbase >= STEPS) {
      load(a, k00, k, last, lane);
      wait_vmcnt<0>();
    }
    return __builtin_amdgcn_readlane(v, (k - kbase) * EPW + r);
  }
};

// wait for vmcnt <= ahead*NL + sg*NS with ahead, sg in [0, NA) x [0, NSG)
template <int NA, int NSG, int NL, int NS>
__device__ __forceinline__ void wait_steps(int ahead, int sg) {
  static_for<NA>([&](auto A) {
    static_for<NSG>([&](auto G) {
      if (ahead == A && sg == G) wait_vmcnt<A * NL + G * NS>();
    });
  });
}

// Launch configuration of a signature / multiplicity: waves per block and
// staging depth, bounded by the 63 outstanding vector-memory operations a wave
// can count and by 64 KB of LDS per workgroup.
template <class S, int U, bool GEOM = false>
struct Cfg {
  using M = LaneMap<U>;
  using R = RecvStage<S, U, GEOM>;
  using Sd = SendStage<S, U, GEOM>;
  // receiver pass stores per step and lane: one word per path and channel set
  // (grad_w), the lane's share of grad_Y after the halving channel sum
  static constexpr int ST_W = S::NP * M::CPL;
  static constexpr int ST_Y = ls_final(GEOM ? 3 : S::YC, M::LPE);   // grad_Y (or grad_r) share
  static constexpr int NST = ST_W + ST_Y;
  // Staging depth: double buffering (deeper pipelines measured slower on the
  // 1,536-atom workload), single buffering when a step has too many memory
  // operations to count or the buffers would exceed the LDS budget.
  static constexpr int depth(int nl, int buf, int waves) {
    return (nl <= 63 && 2 * buf * waves <= 64 * 1024) ? 2 : 1;
  }
  static constexpr bool fits(int buf, int nbuf, int waves) { return buf * nbuf * waves <= 64 * 1024;
  }
  // waves per workgroup of each pass (one if a single buffer per wave for two
  // waves would not fit)
  static constexpr int LDS = 64 * 1024;
  // the forward takes one wave per workgroup up to 32 channels on graphs that
  // fill the chip (no cross-wave reduction; 23.3 against 24.2 us on the
  // 1,536-atom graph with two) and two on small graphs (WPB_F2), where the
  // latency of one workgroup is that of the launch
  // (large signatures take four waves where their single buffers fit: 164
  // against 172 us for the lmax-3 forward, 1.88 against 1.97 ms on the Zipf
  // graph, in node order; at 64 channels and with the nodes in launch order,
  // two: 1.49 against 1.55 ms on the Zipf graph)
  static constexpr int WPB_F2 = 2 * R::BUF <= LDS ? 2 : 1;
  static constexpr int WPB_F = kPhased<S> ? (U == 64 ? 2 : (fits(R::BUF, 1, 4) ? 4 : WPB_F2))
                                          : (U <= 32 ? 1 : WPB_F2);
  // the receiver pass takes four waves where their buffers fit (shorter
  // workgroups that the dispatcher refills as they finish: 39.8 against
  // 42.6 us on the 1,536-atom graph with two); the large signature at 64
  // channels two once the nodes run in launch order (2.79 against 2.89 ms on
  // the Zipf graph)
  static constexpr int WPB_R = (kPhased<S> && U == 64)
                                   ? 2
                                   : (fits(R::BUF, kPhased<S> ? 1 : 2, 4) ? 4 : (2 * R::BUF <= LDS ? 2 : 1));
  // the sender pass one wave per workgroup up to 32 channels and for large
  // signatures (1.73 against 1.86 ms on the Zipf graph with two)
  static constexpr int WPB_S = (U <= 32 || kPhased<S> || 2 * Sd::BUF > LDS) ? 1 : 2;
  // large signatures are arithmetic-heavy: one buffer per wave doubles the
  // workgroups (waves) that fit in LDS, which hides more latency than a
  // second buffer would
  static constexpr int NBUF_F = kPhased<S> ? 1 : depth(R::NLOADS, R::BUF, WPB_F);
  static constexpr int NBUF_F2 = kPhased<S> ? 1 : depth(R::NLOADS, R::BUF, WPB_F2);
  static constexpr int NBUF_R = kPhased<S> ? 1 : depth(R::NLOADS + NST, R::BUF, WPB_R);
  static constexpr int NBUF_S = kPhased<S> ? 1 : depth(Sd::NLOADS, Sd::BUF, WPB_S);
  static_assert(fits(R::BUF, NBUF_F, WPB_F) && fits(R::BUF, NBUF_F2, WPB_F2) && fits(R::BUF, NBUF_R, WPB_R) &&
                    fits(Sd::BUF, NBUF_S, WPB_S), "staging exceeds 64 KB of LDS");
};

template <class S, int U, int WPB, int NBUF, bool GEOM = false>
struct FwdSmem {
  static constexpr int STAGE = NBUF * WPB * RecvStage<S, U, GEOM>::BUF;
  static constexpr int RED = WPB * LaneMap<U>::CPL * S::OC * 65 * 4;
  static constexpr int BYTES = STAGE > RED ? STAGE : RED;
};

// GEOM: Y holds the edge vectors r [E][3] and the harmonics are evaluated on chip.
// EPOS: the edge rows of w and Y are stored in the sender grouping and epos[q]
// is the row of receiver-sorted edge q (otherwise row q itself).
template <class S, int U, int WPB, int NBUF, bool GEOM = false, bool EPOS = false>
__global__ void __launch_bounds__(WPB * 64)
    k_conv_fwd(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col,
               const float* __restrict__ x, const float* __restrict__ Y,
               const float* __restrict__ w, float* __restrict__ out,
               const int32_t* __restrict__ epos, const int32_t* __restrict__ order) {
  using M = LaneMap<U>;
  using T = RecvStage<S, U, GEOM>;
  constexpr int OD = U * S::OC, SLOTS = WPB * M::EPW, EPW = M::EPW;
  static_assert((NBUF - 1) * T::NLOADS < 64, "pipeline too deep for vmcnt");
  __shared__ __attribute__((aligned(16))) char smem[FwdSmem<S, U, WPB, NBUF, GEOM>::BYTES];
  const int i = launch_node(order, gridDim.x);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int slot = lane / M::LPE, uu = lane % M::LPE;
  const int beg = row_ptr[i], end = row_ptr[i + 1];
  const int last = end - 1;
  float acc[M::CPL][S::OC];
#pragma unroll
  for (int cc = 0; cc < M::CPL; ++cc)
#pragma unroll
    for (int o = 0; o < S::OC; ++o) acc[cc][o] = 0.f;
  const int trips = wave_trips<U, WPB>(beg, end, wv);
  char* mybuf = smem + wv * NBUF * T::BUF;
  // first position of this wave (wave-uniform)
  const int q00 = __builtin_amdgcn_readfirstlane(beg + wv * EPW);
  if (trips > 0) {
    IdxWindow<EPW, SLOTS> wj, we;
    wj.load(col, q00, 0, last, lane);
    if constexpr (EPOS) we.load(epos, q00, 0, last, lane);
    int jn[EPW], en[EPW];
    auto stage = [&](char* buf, int q0) {
      if constexpr (EPOS)
        stage_recv_at<S, U, GEOM>(buf, x, Y, w, jn, en, lane);
      else
        stage_recv<S, U, GEOM>(buf, x, Y, w, jn, q0, last, lane);
    };
    auto next = [&](int k) {
#pragma unroll
      for (int r = 0; r < EPW; ++r) {
        jn[r] = wj.get(col, q00, k, r, last, lane);
        if constexpr (EPOS) en[r] = we.get(epos, q00, k, r, last, lane);
      }
    };
    // prologue: stage steps 0 .. NBUF-2
#pragma unroll
    for (int b = 0; b < NBUF - 1; ++b) {
      if (b < trips) {
        next(b);
        stage(mybuf + b * T::BUF, q00 + b * SLOTS);
      }
    }
    next(NBUF - 1);
    for (int k = 0; k < trips; ++k) {
      const int q0 = q00 + k * SLOTS;
      const char* cur = mybuf + (k % NBUF) * T::BUF;
      int ahead = trips - 1 - k;
      if (ahead >= NBUF - 1) {
        ahead = NBUF - 1;
        stage(mybuf + ((k + NBUF - 1) % NBUF) * T::BUF, q0 + (NBUF - 1) * SLOTS);
      }
      wait_steps<NBUF, 1, T::NLOADS, 0>(ahead, 0);
      float xr[M::CPL][S::XC], yr[S::YC], wr[M::CPL][S::NP], geo[4];
      read_recv<S, U, GEOM>(cur, slot, uu, xr, yr, wr, geo);
      __builtin_amdgcn_sched_barrier(0);
      // senders (and edge rows) of the next step to stage
      next(k + NBUF);
      // only the receiver's last step can hold slots past its edges (they
      // re-read its last edge); their weights are zeroed there alone
      if (q0 + EPW > end) {
        const float m = q0 + slot < end ? 1.f : 0.f;
#pragma unroll
        for (int cc = 0; cc < M::CPL; ++cc)
#pragma unroll
          for (int p = 0; p < S::NP; ++p) wr[cc][p] *= m;
      }
#pragma unroll
      for (int cc = 0; cc < M::CPL; ++cc) edge_fwd<S>(xr[cc], yr, wr[cc], acc[cc]);
    }
  }
  __syncthreads();   // staging buffers become the reduction buffer
  block_reduce_store<U, WPB, S::OC, S::NO>(acc, (float*)smem, out + (size_t)i * OD, OutBlocks<S>{});
}

// MODE bit 0: write grad_w; bit 1: write grad_Y (with GEOM: Y holds the edge
// vectors r [E][3] and grad_Y receives grad_r [E][3])
template <class S, int U, int WPB, int NBUF, int MODE, bool GEOM = false>
__global__ void __launch_bounds__(WPB * 64)
    k_conv_bwd_recv(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col,
                    const float* __restrict__ x, const float* __restrict__ Y,
                    const float* __restrict__ w, const float* __restrict__ g,
                    float* __restrict__ grad_w, float* __restrict__ grad_Y,
                    const int32_t* __restrict__ order) {
  using M = LaneMap<U>;
  using T = RecvStage<S, U, GEOM>;
  using C = Cfg<S, U, GEOM>;
  constexpr int OD = U * S::OC, SLOTS = WPB * M::EPW, EPW = M::EPW;
  constexpr int NST = ((MODE & 1) ? C::ST_W : 0) + ((MODE & 2) ? C::ST_Y : 0);
  static_assert((NBUF - 1) * (T::NLOADS + NST) < 64, "pipeline too deep for vmcnt");
  constexpr int WAVE_LDS = NBUF * T::BUF;
  __shared__ __attribute__((aligned(16))) char smem[WPB * WAVE_LDS];
  const int i = launch_node(order, gridDim.x);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int slot = lane / M::LPE, uu = lane % M::LPE;
  const int beg = row_ptr[i], end = row_ptr[i + 1];
  const int last = end - 1;
  const int trips = wave_trips<U, WPB>(beg, end, wv);
  if (trips == 0) return;
  const int q00 = __builtin_amdgcn_readfirstlane(beg + wv * EPW);
  IdxWindow<EPW, SLOTS> wj;
  wj.load(col, q00, 0, last, lane);
  float gr[M::CPL][S::OC];
  load_orow<S, U>(g + (size_t)i * OD, uu, gr);
  // grad_out (and the senders) must have landed before the pipelined loop
  // starts: a wait for them inside the loop would also wait for the staging
  // loads in flight
  wait_vmcnt<0>();
  char* mybuf = smem + wv * WAVE_LDS;
  int jn[EPW];
#pragma unroll
  for (int b = 0; b < NBUF - 1; ++b) {
    if (b < trips) {
#pragma unroll
      for (int r = 0; r < EPW; ++r) jn[r] = wj.get(col, q00, b, r, last, lane);
      stage_recv<S, U, GEOM>(mybuf + b * T::BUF, x, Y, w, jn, q00 + b * SLOTS, last, lane);
    }
  }
#pragma unroll
  for (int r = 0; r < EPW; ++r) jn[r] = wj.get(col, q00, NBUF - 1, r, last, lane);
  // Results of step k are stored during step k+1, after its wait, straight
  // from registers; the number of store instructions per step is fixed (NST).
  float pgw[M::CPL][S::NP], pgy[C::ST_Y];
  const HalvingShare ysh = halving_share(T::YR, M::LPE, lane);   // this lane's grad_Y (grad_r) components
  size_t pq = 0;
  auto flush = [&]() {
    if constexpr (MODE & 1) {
#pragma unroll
      for (int cc = 0; cc < M::CPL; ++cc)
#pragma unroll
        for (int p = 0; p < S::NP; ++p)
          __builtin_nontemporal_store(pgw[cc][p], grad_w + (pq * S::NP + p) * U + uu + 64 * cc);
    }
    if constexpr (MODE & 2) {
#pragma unroll
      for (int r = 0; r < C::ST_Y; ++r)
        if (r < ysh.len) __builtin_nontemporal_store(pgy[r], grad_Y + pq * T::YR + ysh.first + r);
    }
  };
  for (int k = 0; k < trips; ++k) {
    const int q0 = q00 + k * SLOTS;
    const char* cur = mybuf + (k % NBUF) * T::BUF;
    int ahead = trips - 1 - k;
    if (ahead >= NBUF - 1) {
      ahead = NBUF - 1;
      stage_recv<S, U, GEOM>(mybuf + ((k + NBUF - 1) % NBUF) * T::BUF, x, Y, w, jn,
                             q0 + (NBUF - 1) * SLOTS, last, lane);
    }
    // store groups issued after this step's loads: steps max(1, k-NBUF+1) .. k-1
    const int sg = k - 1 < NBUF - 1 ? (k - 1 > 0 ? k - 1 : 0) : NBUF - 1;
    wait_steps<NBUF, NBUF, T::NLOADS, NST>(ahead, sg);
    if (k > 0) flush();
    float xr[M::CPL][S::XC], yr[S::YC], wr[M::CPL][S::NP], geo[4];
    read_recv<S, U, GEOM>(cur, slot, uu, xr, yr, wr, geo);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < EPW; ++r) jn[r] = wj.get(col, q00, k + NBUF, r, last, lane);
    float gy[S::YC];
#pragma unroll
    for (int b = 0; b < S::YC; ++b) gy[b] = 0.f;
#pragma unroll
    for (int cc = 0; cc < M::CPL; ++cc) edge_bwd_recv<S>(xr[cc], yr, wr[cc], gr[cc], pgw[cc], gy);
    // sum over the edge's channel lanes (partners stay inside the slot); the
    // lane then holds components ysh.first .. ysh.first + ysh.len - 1
    if constexpr (MODE & 2) edge_grad_share<S, GEOM, M::LPE>(gy, geo, lane, pgy);
    pq = (size_t)min(q0 + slot, last);
  }
  flush();
}

template <class S, int U, int WPB, int NBUF, bool GEOM = false>
struct SendSmem {
  static constexpr int STAGE = NBUF * WPB * SendStage<S, U, GEOM>::BUF;
  static constexpr int RED = WPB * LaneMap<U>::CPL * S::XC * 65 * 4;
  static constexpr int BYTES = STAGE > RED ? STAGE : RED;
};

// GEOM: Y holds the edge vectors r [E][3] and the harmonics are evaluated on chip
template <class S, int U, int WPB, int NBUF, bool GEOM = false>
__global__ void __launch_bounds__(WPB * 64)
    k_conv_bwd_send(const int32_t* __restrict__ t_row_ptr, const int32_t* __restrict__ t_perm,
                    const int32_t* __restrict__ t_col, const float* __restrict__ Y,
                    const float* __restrict__ w, const float* __restrict__ g,
                    float* __restrict__ grad_x, const int32_t* __restrict__ order) {
  using M = LaneMap<U>;
  using T = SendStage<S, U, GEOM>;
  constexpr int XD = U * S::XC, SLOTS = WPB * M::EPW, EPW = M::EPW;
  static_assert((NBUF - 1) * T::NLOADS < 64, "pipeline too deep for vmcnt");
  __shared__ __attribute__((aligned(16))) char smem[SendSmem<S, U, WPB, NBUF, GEOM>::BYTES];
  const int j = launch_node(order, gridDim.x);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int slot = lane / M::LPE, uu = lane % M::LPE;
  const int beg = t_row_ptr[j], end = t_row_ptr[j + 1];
  const int last = end - 1;
  float gx[M::CPL][S::XC];
#pragma unroll
  for (int cc = 0; cc < M::CPL; ++cc)
#pragma unroll
    for (int a = 0; a < S::XC; ++a) gx[cc][a] = 0.f;
  const int trips = wave_trips<U, WPB>(beg, end, wv);
  char* mybuf = smem + wv * NBUF * T::BUF;
  const int k00 = __builtin_amdgcn_readfirstlane(beg + wv * EPW);
  if (trips > 0) {
    IdxWindow<EPW, SLOTS> wq, wi;
    wq.load(t_perm, k00, 0, last, lane);
    wi.load(t_col, k00, 0, last, lane);
    int qn[EPW], in[EPW];
#pragma unroll
    for (int b = 0; b < NBUF - 1; ++b) {
      if (b < trips) {
#pragma unroll
        for (int r = 0; r < EPW; ++r) {
          qn[r] = wq.get(t_perm, k00, b, r, last, lane);
          in[r] = wi.get(t_col, k00, b, r, last, lane);
        }
        stage_send<S, U, GEOM>(mybuf + b * T::BUF, Y, w, g, qn, in, lane);
      }
    }
#pragma unroll
    for (int r = 0; r < EPW; ++r) {
      qn[r] = wq.get(t_perm, k00, NBUF - 1, r, last, lane);
      in[r] = wi.get(t_col, k00, NBUF - 1, r, last, lane);
    }
    for (int k = 0; k < trips; ++k) {
      const int k0 = k00 + k * SLOTS;
      const char* cur = mybuf + (k % NBUF) * T::BUF;
      int ahead = trips - 1 - k;
      if (ahead >= NBUF - 1) {
        ahead = NBUF - 1;
        stage_send<S, U, GEOM>(mybuf + ((k + NBUF - 1) % NBUF) * T::BUF, Y, w, g, qn, in, lane);
      }
      wait_steps<NBUF, 1, T::NLOADS, 0>(ahead, 0);
      const float* W = (const float*)(cur + T::W_OFF) + slot * (S::NP * U);
      const float* Yv = (const float*)(cur + T::Y_OFF) + slot * T::YR;
      const float* G = (const float*)(cur + T::G_OFF) + slot * (S::OC * U);
      float yr[S::YC], wr[M::CPL][S::NP], gr[M::CPL][S::OC], geo[4];
      read_y<S, GEOM>(Yv, yr, geo);
#pragma unroll
      for (int cc = 0; cc < M::CPL; ++cc) {
#pragma unroll
        for (int p = 0; p < S::NP; ++p) wr[cc][p] = W[p * U + uu + 64 * cc];
        static_for<S::NO>([&](auto K) {
          constexpr OutInfo oi = S::outs.o[K];
          constexpr int d = 2 * oi.l + 1;
          const float* pg = G + U * oi.ko + (uu + 64 * cc) * d;
          static_for<d>([&](auto C) { gr[cc][oi.ko + C] = pg[C]; });
        });
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < EPW; ++r) {
        qn[r] = wq.get(t_perm, k00, k + NBUF, r, last, lane);
        in[r] = wi.get(t_col, k00, k + NBUF, r, last, lane);
      }
      // only the sender's last step can hold slots past its edges
      if (k0 + EPW > end) {
        const float m = k0 + slot < end ? 1.f : 0.f;
#pragma unroll
        for (int cc = 0; cc < M::CPL; ++cc)
#pragma unroll
          for (int p = 0; p < S::NP; ++p) wr[cc][p] *= m;
      }
#pragma unroll
      for (int cc = 0; cc < M::CPL; ++cc) edge_bwd_send<S>(yr, wr[cc], gr[cc], gx[cc]);
    }
  }
  __syncthreads();
  block_reduce_store<U, WPB, S::XC, S::NIN>(gx, (float*)smem, grad_x + (size_t)j * XD, InBlocks<S>{});
}

// ---------------------------------------------------------------------------
// Whole backward in one sender-grouped pass.
//
// A workgroup owns sender j with x[j] in registers and walks its edges in the
// sender grouping; per edge e = (j -> i) it stages w[e], Y[e] and grad_out[i]
// and forms all three gradients from them:
//   grad_w[e] and grad_Y[e] exactly as the receiver pass (Z form), stored at
//   the edge's receiver-sorted position q = t_perm[k] (rows of P*U weights
//   stay whole, so the stores are full cache lines);
//   grad_x[j] accumulated in registers as the sender pass does.
// So w and Y are read once per backward and grad_out is the only gathered
// operand ("Sobek", Abstract: the backward consumes edge-local products into
// bounded node-side state; no edge-sized adjoint beyond the requested
// grad_w / grad_Y).  A slot past the sender's edges works on its clamped
// last edge: its grad_w / grad_Y equal the real slot's bit for bit (same
// operands, same lane arithmetic), and its grad_x share is masked.
// Results of step k are stored during step k+1, after its wait.
// MODE bit 0: write grad_w; bit 1: write grad_Y.
template <class S, int U, bool GEOM = false>
struct FusedCfg {
  using Sd = SendStage<S, U, GEOM>;
  using C = Cfg<S, U, GEOM>;
  // four waves per sender, two staging buffers each (about 70 KB per
  // workgroup at 32 channels: two workgroups share a compute unit's 160 KB);
  // measured on the 1,536-atom graph against 1 to 4 waves and 1 to 3 buffers,
  // which all land within 10 %: the pass moves about as many bytes per second
  // as a plain device copy
  static constexpr int NBUF = 2;
  static constexpr int WPB = (4 * NBUF * Sd::BUF <= 80 * 1024) ? 4 : (2 * NBUF * Sd::BUF <= 80 * 1024 ? 2 : 1);
};

template <class S, int U, int WPB, int NBUF, bool GEOM = false>
struct FusedSmem {
  static constexpr int XB = S::XC * U * 4;                      // the sender's x row, per wave
  static constexpr int XR_OFF = NBUF * WPB * SendStage<S, U, GEOM>::BUF;
  static constexpr int STAGE = XR_OFF + WPB * ceil16(XB);
  static constexpr int RED = WPB * LaneMap<U>::CPL * S::XC * 65 * 4;
  static constexpr int BYTES = STAGE > RED ? STAGE : RED;
};

// GEOM: Y holds the edge vectors r [E][3] and grad_Y receives grad_r [E][3].
// IDQ: the edge rows (w, Y, grad_w, grad_Y) are stored in the sender grouping,
// so the row of sender-grouped position k is k itself and t_perm is not read.
// grad_x may be null (not stored).
template <class S, int U, int WPB, int NBUF, int MODE, bool GEOM = false, bool IDQ = false>
__global__ void __launch_bounds__(WPB * 64)
    k_conv_bwd_fused(const int32_t* __restrict__ t_row_ptr, const int32_t* __restrict__ t_perm,
                     const int32_t* __restrict__ t_col, const float* __restrict__ x,
                     const float* __restrict__ Y, const float* __restrict__ w,
                     const float* __restrict__ g, float* __restrict__ grad_x,
                     float* __restrict__ grad_w, float* __restrict__ grad_Y,
                     const int32_t* __restrict__ order) {
  using M = LaneMap<U>;
  using T = SendStage<S, U, GEOM>;
  using C = Cfg<S, U, GEOM>;
  using SM = FusedSmem<S, U, WPB, NBUF, GEOM>;
  constexpr int XD = U * S::XC, SLOTS = WPB * M::EPW, EPW = M::EPW;
  constexpr int NST = ((MODE & 1) ? C::ST_W : 0) + ((MODE & 2) ? C::ST_Y : 0);
  static_assert(NBUF >= 1 && NBUF <= 4, "one to four staging buffers");
  static_assert((NBUF - 1) * (T::NLOADS + NST) < 64, "pipeline too deep for vmcnt");
  __shared__ __attribute__((aligned(16))) char smem[SM::BYTES];
  const int j = launch_node(order, gridDim.x);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int slot = lane / M::LPE, uu = lane % M::LPE;
  const int beg = t_row_ptr[j], end = t_row_ptr[j + 1];
  const int last = end - 1;
  float gx[M::CPL][S::XC];
#pragma unroll
  for (int cc = 0; cc < M::CPL; ++cc)
#pragma unroll
    for (int a = 0; a < S::XC; ++a) gx[cc][a] = 0.f;
  const int trips = wave_trips<U, WPB>(beg, end, wv);
  char* mybuf = smem + wv * NBUF * T::BUF;
  char* myx = smem + SM::XR_OFF + wv * ceil16(SM::XB);
  const int k00 = __builtin_amdgcn_readfirstlane(beg + wv * EPW);
  if (trips > 0) {
    // the sender's x row goes to LDS ahead of the first step's operands, so
    // the first step's wait covers it (loads complete in issue order)
    dma_rows16<1, SM::XB>(myx, [&](int) { return (const char*)(x + (size_t)j * XD); }, lane);
    // qh[t]: receiver-sorted positions of the steps staged but not yet
    // computed (qh[0] is the next one computed); qn/in: the step staged next
    IdxWindow<EPW, SLOTS> wq, wi;
    if constexpr (!IDQ) wq.load(t_perm, k00, 0, last, lane);
    wi.load(t_col, k00, 0, last, lane);
    // row of the edge in slot r at wave step t
    auto row_at = [&](int t, int r) {
      if constexpr (IDQ)
        return min(k00 + t * SLOTS + r, last);
      else
        return wq.get(t_perm, k00, t, r, last, lane);
    };
    int qh[NBUF > 1 ? NBUF - 1 : 1][EPW], qn[EPW], in[EPW];
#pragma unroll
    for (int b = 0; b < NBUF - 1; ++b) {
#pragma unroll
      for (int r = 0; r < EPW; ++r) {
        qn[r] = row_at(b, r);
        in[r] = wi.get(t_col, k00, b, r, last, lane);
        qh[b][r] = qn[r];
      }
      if (b < trips) stage_send<S, U, GEOM>(mybuf + b * T::BUF, Y, w, g, qn, in, lane);
    }
#pragma unroll
    for (int r = 0; r < EPW; ++r) {
      qn[r] = row_at(NBUF - 1, r);
      in[r] = wi.get(t_col, k00, NBUF - 1, r, last, lane);
    }
    float xr[M::CPL][S::XC];
    float pgw[M::CPL][S::NP], pgy[C::ST_Y];
    const HalvingShare ysh = halving_share(T::YR, M::LPE, lane);
    size_t pq = 0;
    auto flush = [&]() {
      if constexpr (MODE & 1) {
#pragma unroll
        for (int cc = 0; cc < M::CPL; ++cc)
#pragma unroll
          for (int p = 0; p < S::NP; ++p)
            __builtin_nontemporal_store(pgw[cc][p], grad_w + (pq * S::NP + p) * U + uu + 64 * cc);
      }
      if constexpr (MODE & 2) {
#pragma unroll
        for (int r = 0; r < C::ST_Y; ++r)
          if (r < ysh.len) __builtin_nontemporal_store(pgy[r], grad_Y + pq * T::YR + ysh.first + r);
      }
    };
    for (int k = 0; k < trips; ++k) {
      const int k0 = k00 + k * SLOTS;
      const char* cur = mybuf + (k % NBUF) * T::BUF;
      // receiver-sorted position of this lane's edge
      const int q = NBUF == 1 ? pick(qn, slot) : pick(qh[0], slot);
      int ahead = trips - 1 - k;
      if (ahead >= NBUF - 1) {
        ahead = NBUF - 1;
        stage_send<S, U, GEOM>(mybuf + ((k + NBUF - 1) % NBUF) * T::BUF, Y, w, g, qn, in, lane);
      }
      // store groups issued after this step's loads: steps max(1, k-NBUF+1) .. k-1
      const int sg = k - 1 < NBUF - 1 ? (k - 1 > 0 ? k - 1 : 0) : NBUF - 1;
      wait_steps<NBUF, NBUF, T::NLOADS, NST>(ahead, sg);
      if (k > 0) flush();
      if (k == 0) {
#pragma unroll
        for (int cc = 0; cc < M::CPL; ++cc)
          static_for<S::NIN>([&](auto I) {
            constexpr int d = 2 * S::ls.v[I] + 1;
            constexpr int xo = S::xoff(I);
            const float* px = (const float*)myx + U * xo + (uu + 64 * cc) * d;
            static_for<d>([&](auto A) { xr[cc][xo + A] = px[A]; });
          });
      }
      const float* W = (const float*)(cur + T::W_OFF) + slot * (S::NP * U);
      const float* Yv = (const float*)(cur + T::Y_OFF) + slot * T::YR;
      const float* G = (const float*)(cur + T::G_OFF) + slot * (S::OC * U);
      float yr[S::YC], wr[M::CPL][S::NP], gr[M::CPL][S::OC], geo[4];
      read_y<S, GEOM>(Yv, yr, geo);
#pragma unroll
      for (int cc = 0; cc < M::CPL; ++cc) {
#pragma unroll
        for (int p = 0; p < S::NP; ++p) wr[cc][p] = W[p * U + uu + 64 * cc];
        static_for<S::NO>([&](auto K) {
          constexpr OutInfo oi = S::outs.o[K];
          constexpr int d = 2 * oi.l + 1;
          const float* pg = G + U * oi.ko + (uu + 64 * cc) * d;
          static_for<d>([&](auto Cc) { gr[cc][oi.ko + Cc] = pg[Cc]; });
        });
      }
      __builtin_amdgcn_sched_barrier(0);
      // positions of the steps still in flight, and indices of the step
      // after the staged one, loaded while this step computes
      if constexpr (NBUF > 1) {
#pragma unroll
        for (int t = 0; t + 1 < NBUF - 1; ++t)
#pragma unroll
          for (int r = 0; r < EPW; ++r) qh[t][r] = qh[t + 1][r];
#pragma unroll
        for (int r = 0; r < EPW; ++r) qh[NBUF - 2][r] = qn[r];
      }
#pragma unroll
      for (int r = 0; r < EPW; ++r) {
        qn[r] = row_at(k + NBUF, r);
        in[r] = wi.get(t_col, k00, k + NBUF, r, last, lane);
      }
      float gy[S::YC];
#pragma unroll
      for (int b = 0; b < S::YC; ++b) gy[b] = 0.f;
      // only the sender's last step can hold slots past its edges; their
      // grad_x share is dropped (their grad_w / grad_Y are the real slot's)
      const bool live = k0 + slot < end;
      if constexpr (!kPhased<S>) {
        float ym[S::YC];
#pragma unroll
        for (int b = 0; b < S::YC; ++b) ym[b] = live ? yr[b] : 0.f;
#pragma unroll
        for (int cc = 0; cc < M::CPL; ++cc) edge_bwd_all<S>(xr[cc], yr, ym, wr[cc], gr[cc], pgw[cc], gy, gx[cc]);
      } else {
#pragma unroll
        for (int cc = 0; cc < M::CPL; ++cc) edge_bwd_recv<S>(xr[cc], yr, wr[cc], gr[cc], pgw[cc], gy);
        if (k0 + EPW > end) {
#pragma unroll
          for (int cc = 0; cc < M::CPL; ++cc)
#pragma unroll
            for (int c = 0; c < S::OC; ++c) gr[cc][c] = live ? gr[cc][c] : 0.f;
        }
#pragma unroll
        for (int cc = 0; cc < M::CPL; ++cc) edge_bwd_send<S>(yr, wr[cc], gr[cc], gx[cc]);
      }
      if constexpr (MODE & 2) edge_grad_share<S, GEOM, M::LPE>(gy, geo, lane, pgy);
      pq = (size_t)q;
    }
    flush();
  }
  if (!grad_x) return;
  __syncthreads();
  block_reduce_store<U, WPB, S::XC, S::NIN>(gx, (float*)smem, grad_x + (size_t)j * XD, InBlocks<S>{});
}

// ---------------------------------------------------------------------------
// launchers

// below this many receivers (four per compute unit) a launch does not fill the
// chip and the forward takes more waves per receiver
constexpr int kSmallGraph = 1024;

// GEOM: the edge operand is r (a.r) instead of Y, and the edge gradient grad_r
// (a.grad_r) instead of grad_Y
template <bool GEOM>
const float* edge_geom(const ConvArgs& a) {
  return GEOM ? a.r : a.Y;
}
template <bool GEOM>
float* edge_geom_grad(const ConvArgs& a) {
  return GEOM ? a.grad_r : a.grad_Y;
}

template <class S, int U, bool GEOM = false, bool EPOS = false>
hipError_t launch_fwd_as(const ConvArgs& a) {
  using C = Cfg<S, U, GEOM>;
  const float* Y = edge_geom<GEOM>(a);
  if constexpr (C::WPB_F != C::WPB_F2) {
    if (a.n_nodes < kSmallGraph) {
      hipLaunchKernelGGL((k_conv_fwd<S, U, C::WPB_F2, C::NBUF_F2, GEOM, EPOS>), dim3(a.n_nodes),
                         dim3(C::WPB_F2 * 64), 0, a.stream, a.row_ptr, a.col, a.x, Y, a.w, a.out, a.e_pos, a.r_order);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((k_conv_fwd<S, U, C::WPB_F, C::NBUF_F, GEOM, EPOS>), dim3(a.n_nodes), dim3(C::WPB_F * 64), 0,
                     a.stream, a.row_ptr, a.col, a.x, Y, a.w, a.out, a.e_pos, a.r_order);
  return hipGetLastError();
}

// edge rows in receiver-sorted order, or (a.sender_rows, direct-weight form
// only) in the sender grouping, read through a.e_pos
template <class S, int U, bool GEOM = false>
hipError_t launch_fwd(const ConvArgs& a) {
  if (a.n_nodes == 0) return hipSuccess;
  if constexpr (!GEOM) {
    if (a.sender_rows) return launch_fwd_as<S, U, false, true>(a);
  }
  return launch_fwd_as<S, U, GEOM, false>(a);
}

template <class S, int U, bool GEOM = false>
hipError_t launch_bwd_recv(const ConvArgs& a) {
  using C = Cfg<S, U, GEOM>;
  const float* Y = edge_geom<GEOM>(a);
  float* gY = edge_geom_grad<GEOM>(a);
  if (a.n_nodes == 0 || a.n_edges == 0 || (!a.grad_w && !gY)) return hipSuccess;
  const dim3 grid(a.n_nodes), block(C::WPB_R * 64);
  if (a.grad_w && gY)
    hipLaunchKernelGGL((k_conv_bwd_recv<S, U, C::WPB_R, C::NBUF_R, 3, GEOM>), grid, block, 0, a.stream,
                       a.row_ptr, a.col, a.x, Y, a.w, a.grad_out, a.grad_w, gY, a.r_order);
  else if (a.grad_w)
    hipLaunchKernelGGL((k_conv_bwd_recv<S, U, C::WPB_R, C::NBUF_R, 1, GEOM>), grid, block, 0, a.stream,
                       a.row_ptr, a.col, a.x, Y, a.w, a.grad_out, a.grad_w, gY, a.r_order);
  else
    hipLaunchKernelGGL((k_conv_bwd_recv<S, U, C::WPB_R, C::NBUF_R, 2, GEOM>), grid, block, 0, a.stream,
                       a.row_ptr, a.col, a.x, Y, a.w, a.grad_out, a.grad_w, gY, a.r_order);
  return hipGetLastError();
}

template <class S, int U, bool GEOM = false>
hipError_t launch_bwd_send(const ConvArgs& a) {
  using C = Cfg<S, U, GEOM>;
  if (a.n_nodes == 0 || !a.grad_x) return hipSuccess;
  hipLaunchKernelGGL((k_conv_bwd_send<S, U, C::WPB_S, C::NBUF_S, GEOM>), dim3(a.n_nodes), dim3(C::WPB_S * 64),
                     0, a.stream, a.t_row_ptr, a.t_perm, a.t_col, edge_geom<GEOM>(a), a.w, a.grad_out,
                     a.grad_x, a.s_order);
  return hipGetLastError();
}

// whole backward (grad_x with grad_w and/or grad_Y) in one sender-grouped pass

template <class S, int U, bool GEOM = false, bool IDQ = false>
hipError_t launch_bwd_fused_as(const ConvArgs& a) {
  using F = FusedCfg<S, U, GEOM>;
  const float* Y = edge_geom<GEOM>(a);
  float* gY = edge_geom_grad<GEOM>(a);
  const dim3 grid(a.n_nodes), block(F::WPB * 64);
  if (a.grad_w && gY)
    hipLaunchKernelGGL((k_conv_bwd_fused<S, U, F::WPB, F::NBUF, 3, GEOM, IDQ>), grid, block, 0, a.stream,
                       a.t_row_ptr, a.t_perm, a.t_col, a.x, Y, a.w, a.grad_out, a.grad_x, a.grad_w, gY, a.s_order);
  else if (a.grad_w)
    hipLaunchKernelGGL((k_conv_bwd_fused<S, U, F::WPB, F::NBUF, 1, GEOM, IDQ>), grid, block, 0, a.stream,
                       a.t_row_ptr, a.t_perm, a.t_col, a.x, Y, a.w, a.grad_out, a.grad_x, a.grad_w, gY, a.s_order);
  else if (gY)
    hipLaunchKernelGGL((k_conv_bwd_fused<S, U, F::WPB, F::NBUF, 2, GEOM, IDQ>), grid, block, 0, a.stream,
                       a.t_row_ptr, a.t_perm, a.t_col, a.x, Y, a.w, a.grad_out, a.grad_x, a.grad_w, gY, a.s_order);
  else if constexpr (IDQ)
    hipLaunchKernelGGL((k_conv_bwd_fused<S, U, F::WPB, F::NBUF, 0, GEOM, IDQ>), grid, block, 0, a.stream,
                       a.t_row_ptr, a.t_perm, a.t_col, a.x, Y, a.w, a.grad_out, a.grad_x, a.grad_w, gY, a.s_order);
  return hipGetLastError();
}

// edge rows in receiver-sorted order (gathered through t_perm), or
// (a.sender_rows, direct-weight form only) already in the sender grouping; in
// that layout this pass serves any subset of grad_x, grad_w and grad_Y
template <class S, int U, bool GEOM = false>
hipError_t launch_bwd_fused(const ConvArgs& a) {
  if (a.n_nodes == 0) return hipSuccess;
  if constexpr (!GEOM) {
    if (a.sender_rows) return launch_bwd_fused_as<S, U, false, true>(a);
  }
  return launch_bwd_fused_as<S, U, GEOM, false>(a);
}

// Backward of the edge-vector form: grad_x, grad_w and grad_r (a.r, a.grad_r),
// one sender-grouped pass where the signature has it and both kinds of
// gradient are asked for, else a receiver pass and a sender pass.
template <class S, int U>
hipError_t launch_bwd_geom(const ConvArgs& a) {
  const bool edge = a.grad_w || a.grad_r;
  if constexpr (!kPhased<S>) {
    if (a.grad_x && edge && a.n_edges > 0) return launch_bwd_fused<S, U, true>(a);
  }
  hipError_t e = launch_bwd_recv<S, U, true>(a);
  if (e != hipSuccess) return e;
  return launch_bwd_send<S, U, true>(a);
}

}  // namespace tpc

#include "dbl_kernels.hpp"

namespace tpc {

// The one-pass backward where its per-edge arithmetic fits in registers
// (lmax 2); the large signatures are bound by their CG arithmetic and keep the
// two passes (Zipf backward 5.0 against 6.0 ms in one pass).
template <class S, int U>
constexpr LaunchFn fused_backward() {
  if constexpr (kPhased<S>)
    return nullptr;
  else
    return &launch_bwd_fused<S, U>;
}

template <class S, int U>
const KernelSet* kernel_set() {
  static const KernelSet k{&launch_fwd<S, U>,      &launch_bwd_recv<S, U>, &launch_bwd_send<S, U>,
                           &launch_dbl_recv<S, U>, &launch_dbl_send<S, U>, fused_backward<S, U>(),
                           &launch_fwd<S, U, true>, &launch_bwd_geom<S, U>};
  return &k;
}

}  // namespace tpc
