// Tensor-product convolution whose edge weights come from a radial network of
// the edge length, computed on chip and never stored.
//
// The pages reassociate the radial projection with the coupling and the
// aggregation so that per-edge weights do not exist in memory ("Sobek:
// Streaming Equivariant Tensor Product Convolutions", Abstract and AI
// Summary).  Network (reading of the pages, which do not define it):
//   B_n(r) = sqrt(2/r_c) sin(n pi r / r_c) / r,  n = 1..NB
//   h = SiLU(B W1)            W1: [NB][NH]
//   w[e, p, u] = (h W2)[p*U + u]   W2: [NH][P*U]
//
// The layer h -> w is a dense [edges x NH] x [NH x P*U] contraction and runs on
// fp32 MFMA (v_mfma_f32_16x16x4f32).  Operand layout (wave64): lane l supplies
// A[l%16][l/16], B[l/16][l%16] and holds D[4(l/16)+i][l%16].  An M-tile is 16
// edges; an N-tile is one path for 16 consecutive channels, so after the NH/4
// K-steps lane l holds w[edge 4(l/16)+i][p][channel l%16] for every path p --
// exactly the operands the per-lane tensor-product arithmetic needs, with no
// shuffle.  The weights of a chunk of 16 channels live only in registers.
#pragma once
#include "conv_kernels.hpp"

namespace tpc {

// An edge's harmonics and length: read from Y [E][(lmax+1)^2] and r_len [E],
// or, with GEOM, evaluated from the edge vector r [E][3] (passed as Y).
template <class S, bool GEOM>
__device__ __forceinline__ void radial_edge_y(const float* __restrict__ Y, size_t e, float (&yr)[S::YC]) {
  if constexpr (GEOM) {
    float x = Y[3 * e], y = Y[3 * e + 1], z = Y[3 * e + 2], inv;
    unit_dir(x, y, z, inv);
    sh_eval<S::lmax_sh>(x, y, z, yr);
  } else {
#pragma unroll
    for (int t = 0; t < S::YC; ++t) yr[t] = Y[e * S::YC + t];
  }
}
template <bool GEOM>
__device__ __forceinline__ float radial_edge_len(const float* __restrict__ Y, const float* __restrict__ r_len,
                                                 size_t e) {
  if constexpr (GEOM) {
    float x = Y[3 * e], y = Y[3 * e + 1], z = Y[3 * e + 2], inv;
    return unit_dir(x, y, z, inv);
  } else {
    return r_len[e];
  }
}


typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma_16x16x4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

struct RadialParams {
  float r_cut;
  const float* W1;   // [NB][NH]
  const float* W2;   // [NH][P*U]
};

// logistic function with the hardware exponential and reciprocal (about 1e-6
// relative error, far inside the float32 parity bound); exp overflow gives
// inf and a result of 0, as it should
__device__ __forceinline__ float sigmoid_fast(float z) { return __frcp_rn(1.0f + __expf(-z)); }
__device__ __forceinline__ float silu(float z) { return z * sigmoid_fast(z); }

// x components of channel u of node row j
template <class S, int U>
__device__ __forceinline__ void load_x_channel(const float* __restrict__ x, int j, int u, float (&xr)[S::XC]) {
  const float* row = x + (size_t)j * (U * S::XC);
  static_for<S::NIN>([&](auto I) {
    constexpr int d = 2 * S::ls.v[I] + 1;
    constexpr int xo = S::xoff(I);
    static_for<d>([&](auto A) { xr[xo + A] = row[U * xo + u * d + A]; });
  });
}

// output-like row components of channel u
template <class S, int U>
__device__ __forceinline__ void load_o_channel(const float* __restrict__ g, int i, int u, float (&gr)[S::OC]) {
  const float* row = g + (size_t)i * (U * S::OC);
  static_for<S::NO>([&](auto K) {
    constexpr OutInfo oi = S::outs.o[K];
    constexpr int d = 2 * oi.l + 1;
    static_for<d>([&](auto C) { gr[oi.ko + C] = row[U * oi.ko + u * d + C]; });
  });
}

// The distinct nontrivial coefficient magnitudes (|C| != 1) of one path per
// output component, and for each nonzero the slot of its (c, |C|) (-1 for
// |C| = 1).
template <int L1, int L2, int L3>
struct CgScaled {
  using T = CgPath<L1, L2, L3>;
  struct Tab {
    int c[T::nnz > 0 ? T::nnz : 1];
    float m[T::nnz > 0 ? T::nnz : 1];
    int slot[T::nnz > 0 ? T::nnz : 1];
    int n;
  };
  static constexpr Tab build() {
    Tab t{};
    t.n = 0;
    for (int k = 0; k < T::nnz; ++k) {
      const Nz e = T::table.e[k];
      const float m = e.v < 0.f ? -e.v : e.v;
      if (m == 1.f) {
        t.slot[k] = -1;
        continue;
      }
      int s = -1;
      for (int q = 0; q < t.n; ++q)
        if (t.c[q] == e.c && t.m[q] == m) s = q;
      if (s < 0) {
        s = t.n;
        t.c[t.n] = e.c;
        t.m[t.n] = m;
        ++t.n;
      }
      t.slot[k] = s;
    }
    return t;
  }
  static constexpr Tab tab = build();
};

// z[b] = sum_{a,c} C[a,b,c] x[XO + a] g[GO + c] for one path and one channel,
// the Z-form of the adjoint: g scaled by each distinct nontrivial |C| of the
// path once, then one signed multiply-add per nonzero (instead of forming
// t[b][c] = sum_a C x_a and then z[b] = sum_c t[b][c] g_c)
template <int L1, int L2, int L3, int XO, int GO, int NX, int NG>
__device__ __forceinline__ void zform_scaled(const float (&x)[NX], const float (&g)[NG], float (&z)[2 * L2 + 1]) {
  using T = CgPath<L1, L2, L3>;
  using CS = CgScaled<L1, L2, L3>;
  constexpr int NS = CS::tab.n;
  float gs[NS > 0 ? NS : 1];
  static_for<NS>([&](auto Q) { gs[Q] = CS::tab.m[Q] * g[GO + CS::tab.c[Q]]; });
  static_for<2 * L2 + 1>([&](auto B) { z[B] = 0.f; });
  static_for<T::nnz>([&](auto N) {
    constexpr Nz e = T::table.e[N];
    constexpr int sl = CS::tab.slot[N];
    float gv;
    if constexpr (sl < 0) gv = g[GO + e.c];
    else gv = gs[sl];
    if constexpr (e.v < 0.f) z[e.b] = fmaf(-x[XO + e.a], gv, z[e.b]);
    else z[e.b] = fmaf(x[XO + e.a], gv, z[e.b]);
  });
}

// sum over the four lanes that share l%16 (lanes l, l^16, l^32, l^48)
template <int N>
__device__ __forceinline__ void reduce_quads(float (&v)[N]) {
#pragma unroll
  for (int t = 0; t < N; ++t) {
    v[t] += __shfl_xor(v[t], 16, 64);
    v[t] += __shfl_xor(v[t], 32, 64);
  }
}

// ---------------------------------------------------------------------------
// backward
//
// Receiver pass (grad_Y, grad_W1): the tile is transposed with respect to the
// forward -- M = 16 channels, N = 16 edges -- so lane l owns edge l%16 and the
// four channels 4(l/16)..+3 of the chunk.  The hidden index of K slot (k, l/16)
// is 16(k/4) + 4(l/16) + k%4: with that order the hidden values enter the
// w-MFMA as B operands, grad_w (per path, from the Z-form adjoint) enters the
// grad_h-MFMA as B operands without any shuffle, and the grad_h accumulator
// lands on the lane in the same (edge, hidden) positions as the hidden values,
// so the SiLU derivative is applied in place.

__device__ __forceinline__ int hid_T(int k, int g) { return 16 * (k >> 2) + 4 * g + (k & 3); }

// Hidden values and SiLU derivatives of the edge of lane l (edge l%16 of a
// 16-edge tile) in K-slot order: hB[k] = h[hid_T(k, l/16)].  The
// pre-activations come from a small MFMA, pre^T = W1^T B^T (K = NB), whose D
// layout is exactly that order.  bq[s] = B_{4s + l/16 + 1}(r) is kept for the
// grad_W1 reduction.  Everything is zero for an invalid edge.
// A operands W1[4s + l/16][16t + l%16] of the small MFMA, loaded once per kernel
template <int NB, int NH>
__device__ __forceinline__ void load_w1a(const RadialParams& rp, int e16, int g, float (&w1a)[NH / 16][NB / 4]) {
#pragma unroll
  for (int t = 0; t < NH / 16; ++t)
#pragma unroll
    for (int s = 0; s < NB / 4; ++s) w1a[t][s] = rp.W1[(4 * s + g) * NH + 16 * t + e16];
}

template <int NB, int NH>
__device__ __forceinline__ void hidden_T(float r, bool valid, const RadialParams& rp,
                                         const float (&w1a)[NH / 16][NB / 4], int g,
                                         float (&bq)[NB / 4], float (&hB)[NH / 4], float (&ds)[NH / 4]) {
  static_assert(NB % 4 == 0 && NH % 16 == 0, "hidden tiling");
  const float rr = valid ? r : 1.0f;
  const float pre_b = sqrtf(2.0f / rp.r_cut) / rr;
  const float kk = 3.14159265358979323846f / rp.r_cut;
#pragma unroll
  for (int s = 0; s < NB / 4; ++s) bq[s] = valid ? pre_b * sinf((float)(4 * s + g + 1) * kk * rr) : 0.f;
#pragma unroll
  for (int t = 0; t < NH / 16; ++t) {
    f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NB / 4; ++s) z = mfma_16x16x4(w1a[t][s], bq[s], z);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pre = z[i];
      const float sg = sigmoid_fast(pre);
      hB[4 * t + i] = valid ? pre * sg : 0.f;
      ds[4 * t + i] = valid ? sg * (1.0f + pre * (1.0f - sg)) : 0.f;
    }
  }
}

// channels u0..u0+3 of one node row (u0 a multiple of 4): each irrep block is
// 4(2l+1) consecutive, 16-byte aligned floats
template <class S, int U>
__device__ __forceinline__ void load_x4(const float* __restrict__ x, int j, int u0, float (&xr)[4][S::XC]) {
  const float* row = x + (size_t)j * (U * S::XC);
  static_for<S::NIN>([&](auto I) {
    constexpr int d = 2 * S::ls.v[I] + 1;
    constexpr int xo = S::xoff(I);
    const float4* p = reinterpret_cast<const float4*>(row + U * xo + u0 * d);
    float v[4 * d];
    static_for<d>([&](auto Q) {
      const float4 t = p[Q];
      v[4 * Q + 0] = t.x; v[4 * Q + 1] = t.y; v[4 * Q + 2] = t.z; v[4 * Q + 3] = t.w;
    });
    static_for<4>([&](auto I2) { static_for<d>([&](auto A) { xr[I2][xo + A] = v[I2 * d + A]; }); });
  });
}

// W2 slice of one chunk of 16 channels in LDS: row hid holds, for every path p,
// the 16 floats W2[hid][p*U + 16c .. +15], then 4 floats of padding.  With the
// row stride of NP*16 + 4 floats both operand patterns read conflict-free:
// 16 consecutive floats from four rows 4 apart (A of the w-MFMA), and 16 bytes
// from sixteen consecutive rows (A of the grad_h-MFMA).
template <class S, int NH>
struct W2Slice {
  static constexpr int WS = S::NP * 16 + 4;          // row stride, floats
  static constexpr int FLOATS = NH * WS;
  static constexpr int QUADS = FLOATS / 4;
  static constexpr int BYTES = FLOATS * 4;
};

// cooperative global->LDS copy of chunk c's slice by the NW waves of a workgroup
template <class S, int U, int NH, int NW>
__device__ __forceinline__ void stage_w2(float* w2s, const float* __restrict__ W2, int c, int wv, int lane) {
  using L = W2Slice<S, NH>;
  constexpr int INSTR = (L::QUADS + 64 * NW - 1) / (64 * NW);
  // opaque copy of the lane index: the per-lane source offsets are recomputed
  // per chunk instead of being hoisted into INSTR live 64-bit registers
  asm volatile("" : "+v"(lane));
  static_for<INSTR>([&](auto K) {
    const int blk = K * NW + wv;                    // 64-quad block of this instruction
    const int q = blk * 64 + lane;
    if (blk * 64 < L::QUADS && q < L::QUADS) {
      const int f = 4 * q;
      const int hid = f / L::WS, rem = f - hid * L::WS;
      const int p = rem >> 4;
      const float* src = rem < S::NP * 16 ? W2 + (size_t)hid * (S::NP * U) + p * U + 16 * c + (rem & 15) : W2;
      __builtin_amdgcn_global_load_lds((gbl_void_t*)src, (lds_void_t*)(w2s + blk * 256), 16, 0, 0);
    }
  });
}

// the chunk's 16 channels of grad_out row i into LDS (output blocks back to
// back, each [16][2l+1]); two load instructions per wave
template <class S, int U>
__device__ __forceinline__ void stage_g(float* gs, const float* __restrict__ g, int i, int c, int lane) {
  constexpr int QUADS = 4 * S::OC;                  // 16 * OC floats
  const float* row = g + (size_t)i * (U * S::OC);
  static_for<(QUADS + 63) / 64>([&](auto K) {
    const int q = K * 64 + lane;
    if (q < QUADS) {
      // block of quad q: blocks hold 4(2l+1) quads each, in output order
      int k = 0;
      static_for<S::NO>([&](auto K2) {
        if (q >= 4 * S::outs.o[K2].ko) k = K2;
      });
      int ko = 0, d = 1;
      static_for<S::NO>([&](auto K2) {
        if (k == K2) { ko = S::outs.o[K2].ko; d = 2 * S::outs.o[K2].l + 1; }
      });
      const float* src = row + U * ko + 16 * c * d + (4 * q - 16 * ko);
      __builtin_amdgcn_global_load_lds((gbl_void_t*)src, (lds_void_t*)(gs + K * 256), 16, 0, 0);
    }
  });
}

// Receiver pass.  A workgroup of NW waves walks its receivers tile by tile
// (16 edges of one receiver per wave and round); within a round the waves go
// through the chunks together: the chunk's W2 slice is copied once into LDS
// for all of them, and grad_out of each wave's receiver is staged beside it.
// Per chunk and path: w (MFMA, A from LDS), the Z-form adjoint on VALU
// (grad_w_p, grad_Y += w_p Z_p) and grad_h += W2_p grad_w_p (MFMA).  After the
// chunks: grad_Y is summed over the edge's channel lanes and stored, and
// grad_W1 = B^T (grad_h * SiLU') is reduced through LDS into one partial per
// wave (part[wave][n][hid]), summed later in a fixed order.
// GEOM: Y holds the edge vectors r [E][3] (r_len unused) and grad_Y receives
// grad_r [E][3] = the pullback of grad_Y and grad_rlen to r (grad_rlen unused)
template <class S, int U, int NB, int NH, int NW, bool GEOM = false>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2)))
    k_radial_bwd_recv(int n_nodes, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col,
                      const float* __restrict__ x, const float* __restrict__ Y,
                      const float* __restrict__ r_len, RadialParams rp, const float* __restrict__ gout,
                      float* __restrict__ grad_Y, float* __restrict__ grad_rlen, float* __restrict__ part,
                      const int32_t* __restrict__ order) {
  static_assert(U % 16 == 0 && NH % 16 == 0 && NH <= 64 && NB <= 16, "radial tiling");
  using L = W2Slice<S, NH>;
  constexpr int GF = 16 * S::OC;                    // staged grad_out floats per wave
  constexpr int RED = 16 * (NH + 1) + 16 * NB;      // grad_W1 scratch floats per wave
  static_assert(NW * RED <= L::FLOATS, "grad_W1 scratch reuses the W2 slice");
  __shared__ __attribute__((aligned(16))) float smem[L::FLOATS + NW * GF];
  float* w2s = smem;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int e16 = lane & 15, g = lane >> 4;
  float* gs = smem + L::FLOATS + wv * GF;
  float* red = smem + wv * RED;                     // s_gp [16][NH+1], s_b [16][NB]
  float w1a[NH / 16][NB / 4];
  load_w1a<NB, NH>(rp, e16, g, w1a);
  float w1[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) w1[n] = 0.f;
  // tile cursor of this wave: position pos of the launch order, its receiver i, first edge t0
  const int stride = gridDim.x * NW;
  int pos = blockIdx.x * NW + wv, i = 0, t0 = 0, end = 0;
  auto seek = [&]() {   // first position >= pos whose receiver has edges
    while (pos < n_nodes) {
      i = order ? min(max(order[pos], 0), n_nodes - 1) : pos;
      t0 = row_ptr[i];
      end = row_ptr[i + 1];
      if (t0 < end) break;
      pos += stride;
    }
  };
  seek();
  while (__syncthreads_or(pos < n_nodes)) {
    const bool has = pos < n_nodes;
    const int q = t0 + e16;
    const bool valid = has && q < end;
    const int qc = has ? (q < end ? q : end - 1) : 0;
    const int j = has ? col[qc] : 0;
    float hB[NH / 4], yr[S::YC], gy[S::YC];
    const float rl = has ? radial_edge_len<GEOM>(Y, r_len, qc) : 1.f;
    {
      float bq0[NB / 4], ds0[NH / 4];               // recomputed after the chunks
      hidden_T<NB, NH>(rl, valid, rp, w1a, g, bq0, hB, ds0);
    }
    radial_edge_y<S, GEOM>(Y, qc, yr);              // qc is a valid edge even without a receiver
#pragma unroll
    for (int t = 0; t < S::YC; ++t) {
      yr[t] = has ? yr[t] : 0.f;
      gy[t] = 0.f;
    }
    f32x4 gh[NH / 16];
#pragma unroll
    for (int t = 0; t < NH / 16; ++t) gh[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int c = 0; c < U / 16; ++c) {
      const int u0 = 16 * c + 4 * g;
      __syncthreads();                              // previous chunk's LDS reads done
      stage_w2<S, U, NH, NW>(w2s, rp.W2, c, wv, lane);
      if (has) stage_g<S, U>(gs, gout, i, c, lane);
      float xr[4][S::XC];
      load_x4<S, U>(x, j, u0, xr);
      wait_vmcnt<0>();
      __syncthreads();
      if (has) {
        static_for<S::NP>([&](auto P) {
          constexpr PathInfo pi = S::paths.p[P];
          using T = CgPath<pi.l1, pi.l2, pi.l3>;
          constexpr int D2 = 2 * pi.l2 + 1, D3 = 2 * pi.l3 + 1;
          // w[channel 16c + 4g + r][edge e16]
          const float* wa = w2s + P * 16 + e16;
          f32x4 w = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int k = 0; k < NH / 4; ++k) w = mfma_16x16x4(wa[hid_T(k, g) * L::WS], hB[k], w);
          // grad_out block of the path's output irrep, the lane's four channels
          float gb[4 * D3];
          const float4* gp = reinterpret_cast<const float4*>(gs + 16 * pi.ko + 4 * g * D3);
          static_for<D3>([&](auto Q) {
            const float4 t = gp[Q];
            gb[4 * Q + 0] = t.x; gb[4 * Q + 1] = t.y; gb[4 * Q + 2] = t.z; gb[4 * Q + 3] = t.w;
          });
          float gw[4];
          static_for<4>([&](auto R) {
            float z[D2];
            zform_scaled<pi.l1, pi.l2, pi.l3, pi.xo, R * D3>(xr[R], gb, z);
            float s = 0.f;
            static_for<D2>([&](auto B2) {
              s = fmaf(yr[pi.yo + B2], z[B2], s);
              gy[pi.yo + B2] = fmaf(w[int(R)], z[B2], gy[pi.yo + B2]);
            });
            gw[R] = s;
          });
          // grad_h[hid 16t + 4g + r][edge e16] += sum over the chunk's channels
          const float* wb = w2s + e16 * L::WS + P * 16 + 4 * g;
#pragma unroll
          for (int t = 0; t < NH / 16; ++t) {
            const float4 a4 = *reinterpret_cast<const float4*>(wb + 16 * t * L::WS);
            gh[t] = mfma_16x16x4(a4.x, gw[0], gh[t]);
            gh[t] = mfma_16x16x4(a4.y, gw[1], gh[t]);
            gh[t] = mfma_16x16x4(a4.z, gw[2], gh[t]);
            gh[t] = mfma_16x16x4(a4.w, gw[3], gh[t]);
          }
          __builtin_amdgcn_sched_barrier(0);        // keep each path's temporaries local
        });
      }
    }
    // grad_Y: sum over the four channel groups of the edge
#pragma unroll
    for (int t = 0; t < S::YC; ++t) {
      gy[t] += __shfl_xor(gy[t], 16, 64);
      gy[t] += __shfl_xor(gy[t], 32, 64);
    }
    if (!GEOM && grad_Y && g == 0 && valid) {
#pragma unroll
      for (int t = 0; t < S::YC; ++t) grad_Y[(size_t)q * S::YC + t] = gy[t];
    }
    // The basis values and SiLU derivatives are evaluated again here rather
    // than kept through the chunk loop (their 18 registers would spill); the
    // empty asm hides that the edge length is the same, so the two evaluations
    // are not merged.
    float bq[NB / 4], ds[NH / 4];
    {
      float rl2 = rl, hB2[NH / 4];
      asm volatile("" : "+v"(rl2));
      hidden_T<NB, NH>(rl2, valid, rp, w1a, g, bq, hB2, ds);
    }
    // grad_pre (zero for an invalid edge) in the K-slot order of the hidden values
    float gp[NH / 4];
#pragma unroll
    for (int k = 0; k < NH / 4; ++k) gp[k] = gh[k >> 2][k & 3] * ds[k];
    if ((GEOM ? grad_Y != nullptr : grad_rlen != nullptr) && has) {
      // grad_B[n][edge] = sum_h W1[n][h] grad_pre[h][edge] on the MFMA (rows
      // n >= NB zero); lane l gets n = 4(l/16) + i of edge l%16, then
      // grad_rlen = sum_n grad_B[n] dB_n/dr, summed over the lane groups
      f32x4 gbn = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < NH / 4; ++k)
        gbn = mfma_16x16x4(e16 < NB ? rp.W1[e16 * NH + hid_T(k, g)] : 0.f, gp[k], gbn);
      const float pre_b = sqrtf(2.0f / rp.r_cut), kk = 3.14159265358979323846f / rp.r_cut;
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = 4 * g + i;
        if (n < NB) {
          const float kn = (float)(n + 1) * kk;
          acc += gbn[i] * pre_b * (kn * cosf(kn * rl) / rl - sinf(kn * rl) / (rl * rl));
        }
      }
      acc += __shfl_xor(acc, 16, 64);
      acc += __shfl_xor(acc, 32, 64);
      if constexpr (GEOM) {
        // grad_r = pullback of (grad_Y, grad_rlen) to the edge vector
        if (g == 0 && valid) {
          float ux = Y[3 * (size_t)q], uy = Y[3 * (size_t)q + 1], uz = Y[3 * (size_t)q + 2], inv, o[3];
          unit_dir(ux, uy, uz, inv);
          sh_pullback<S::lmax_sh>(ux, uy, uz, inv, gy, acc, o);
          grad_Y[3 * (size_t)q + 0] = o[0];
          grad_Y[3 * (size_t)q + 1] = o[1];
          grad_Y[3 * (size_t)q + 2] = o[2];
        }
      } else {
        if (g == 0 && valid) grad_rlen[q] = acc;
      }
    }
    // grad_W1[n][hid] += sum over the tile's edges of B_n * grad_pre[hid]
    __syncthreads();                                // W2 slice no longer read
    if (has) {
      float* s_gp = red;
      float* s_b = red + 16 * (NH + 1);
#pragma unroll
      for (int k = 0; k < NH / 4; ++k) s_gp[e16 * (NH + 1) + hid_T(k, g)] = gp[k];
#pragma unroll
      for (int t = 0; t < NB / 4; ++t) s_b[e16 * NB + 4 * t + g] = bq[t];
      __builtin_amdgcn_s_waitcnt(0xc07f);           // lgkmcnt(0): own LDS writes done (one wave)
      __builtin_amdgcn_wave_barrier();
      if (lane < NH) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float gp = s_gp[e * (NH + 1) + lane];
#pragma unroll
          for (int n = 0; n < NB; ++n) w1[n] = fmaf(s_b[e * NB + n], gp, w1[n]);
        }
      }
      // advance the cursor
      t0 += 16;
      if (t0 >= end) {
        pos += stride;
        seek();
      }
    }
  }
  if (lane < NH) {
    float* p = part + (size_t)(blockIdx.x * NW + wv) * (NB * NH);
#pragma unroll
    for (int n = 0; n < NB; ++n) p[n * NH + lane] = w1[n];
  }
}

// grad_W2 pass, chunk-major: workgroup (block, chunk c) of NH/16 waves.  Per
// round every wave takes one 16-edge tile of its receivers and computes the
// Z-form adjoint grad_w of all paths for it (lane l: edges 4(l/16) + r, channel
// 16c + l%16), written to LDS; after a barrier wave w contracts the four
// tiles' grad_w with the hidden values of its own 16 hidden units:
//   grad_W2[hid 16w + .][p*U + 16c + .] += sum over edges of h * grad_w_p
// (MFMA: M = hidden units, N = channels, K = edges).  The hidden values come
// from the small MFMA pre = B W1 (K = NB) whose D layout is the A operand
// needed here, so each wave computes only its own 16 hidden units.  The
// accumulators (one 16x16 tile per path) stay in registers; one partial per
// workgroup is written and summed later in a fixed order.
// GEOM: Y holds the edge vectors r [E][3]; r_len unused.  One launch covers
// the NPG paths P0 .. P0 + NPG - 1 (all paths by default; wider signatures are
// split into groups whose grad_w tiles fit in LDS, one launch per group, each
// writing its own columns of the partials).
template <class S, int U, int NB, int NH, bool GEOM = false, int P0 = 0, int NPG = S::NP>
__global__ void __launch_bounds__(64 * (NH / 16)) __attribute__((amdgpu_waves_per_eu(2)))
    k_radial_bwd_w2(int n_nodes, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col,
                    const float* __restrict__ x, const float* __restrict__ Y,
                    const float* __restrict__ r_len, RadialParams rp, const float* __restrict__ gout,
                    float* __restrict__ part, const int32_t* __restrict__ order) {
  static_assert(U % 16 == 0 && NH % 16 == 0 && NB % 4 == 0, "radial tiling");
  static_assert(P0 >= 0 && NPG > 0 && P0 + NPG <= S::NP, "path group");
  constexpr int NW = NH / 16;
  constexpr int LD = S::NP * U;
  // grad_w of one tile in LDS: [p][edge 16][ch 16 + 4 pad]; the edge-row stride
  // of 20 floats puts the four lane groups (edges 4g + k) on distinct banks
  constexpr int RS = 20, PS = 16 * RS;
  constexpr int TILE = NPG * PS;
  __shared__ __attribute__((aligned(16))) float s_gw[NW * TILE];
  __shared__ float s_r[NW * 16];                    // edge lengths of the tiles (-1: no edge)
  const int c = blockIdx.y;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int e16 = lane & 15, g = lane >> 4;
  const int u = 16 * c + e16;
  f32x4 acc[NPG];
#pragma unroll
  for (int p = 0; p < NPG; ++p) acc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
  // W1 operands of this wave's hidden units (B[n][hid 16w + e16], n = 4s + g)
  float w1b[NB / 4];
#pragma unroll
  for (int s = 0; s < NB / 4; ++s) w1b[s] = rp.W1[(4 * s + g) * NH + 16 * wv + e16];
  const float pre_b = sqrtf(2.0f / rp.r_cut);
  const float kk = 3.14159265358979323846f / rp.r_cut;
  const int stride = gridDim.x * NW;
  int pos = blockIdx.x * NW + wv, i = 0, t0 = 0, end = 0;
  auto seek = [&]() {
    while (pos < n_nodes) {
      i = order ? min(max(order[pos], 0), n_nodes - 1) : pos;
      t0 = row_ptr[i];
      end = row_ptr[i + 1];
      if (t0 < end) break;
      pos += stride;
    }
  };
  seek();
  float* gw_own = s_gw + wv * TILE;
  while (__syncthreads_or(pos < n_nodes)) {
    if (pos < n_nodes) {
      if (g == 0) {
        const int q = t0 + e16;
        s_r[wv * 16 + e16] = q < end ? radial_edge_len<GEOM>(Y, r_len, q) : -1.f;
      }
      float gr[S::OC];
      load_o_channel<S, U>(gout, i, u, gr);
      // grad_w of the lane's four edges, all paths
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int q = t0 + 4 * g + r;
        const int qc = q < end ? q : end - 1;       // its hidden values are zero
        float xr[S::XC], yr[S::YC];
        load_x_channel<S, U>(x, col[qc], u, xr);
        radial_edge_y<S, GEOM>(Y, qc, yr);
        static_for<NPG>([&](auto G) {
          constexpr PathInfo pi = S::paths.p[P0 + G];
          constexpr int D2 = 2 * pi.l2 + 1;
          float z[D2];
          zform_scaled<pi.l1, pi.l2, pi.l3, pi.xo, pi.ko>(xr, gr, z);
          float s = 0.f;
          static_for<D2>([&](auto B2) { s = fmaf(yr[pi.yo + B2], z[B2], s); });
          gw_own[G * PS + (4 * g + r) * RS + e16] = s;
        });
        __builtin_amdgcn_sched_barrier(0);
      }
      t0 += 16;
      if (t0 >= end) {
        pos += stride;
        seek();
      }
    } else {
      // no tile this round: zero lengths and weights-gradients (the latter so
      // that no stale or uninitialised LDS value meets a zero hidden value)
      if (g == 0) s_r[wv * 16 + e16] = -1.f;
      for (int t = lane; t < TILE; t += 64) gw_own[t] = 0.f;
    }
    __syncthreads();
    // contract the tiles of all waves with this wave's hidden units
#pragma unroll 1
    for (int tw = 0; tw < NW; ++tw) {
      const float r = s_r[tw * 16 + e16];
      const bool v = r >= 0.f;
      const float rr = v ? r : 1.0f;
      f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NB / 4; ++s) {
        const float bn = v ? pre_b / rr * sinf((float)(4 * s + g + 1) * kk * rr) : 0.f;
        z = mfma_16x16x4(bn, w1b[s], z);
      }
      // z[i] = pre[edge 4g + i][hid 16w + e16]; h = 0 for an invalid edge
      float hA[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) hA[t] = silu(z[t]);
      const float* gt = s_gw + tw * TILE + 4 * g * RS + e16;
#pragma unroll
      for (int p = 0; p < NPG; ++p)
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[p] = mfma_16x16x4(hA[k], gt[p * PS + k * RS], acc[p]);
    }
    __syncthreads();
  }
  // part[block][hid][p*U + u]; each chunk writes its own columns
  float* pb = part + (size_t)blockIdx.x * NH * LD;
#pragma unroll
  for (int p = 0; p < NPG; ++p)
#pragma unroll
    for (int t = 0; t < 4; ++t) pb[(size_t)(16 * wv + 4 * g + t) * LD + (P0 + p) * U + u] = acc[p][t];
}

// Forward (SEND = false) and sender pass (SEND = true), chunk-major: workgroup
// (block, chunk c) keeps chunk c's W2 slice in LDS for its whole life.  Each
// lane group g (16 lanes, the chunk's 16 channels) of each wave walks its own
// nodes: n = (block*NW + wave)*4 + g, + gridDim.x*NW*4, ..., four edges of its
// node per step.  A step is one 16-edge tile whose rows 4g .. 4g+3 are group
// g's edges: the hidden values come from the small MFMA, the weights of every
// path from the w-MFMA (A = hidden rows of the tile's edges, B = the slice),
// so lane l holds w[edge 4(l/16) + r][channel 16c + l%16], exactly the
// weights of its own group's four edges, and accumulates its node's whole sum
// in registers (a node's edges pad only to a multiple of four, not of 16, and
// no reduction across groups is needed).  Forward: out[i] of receiver i
// (edges grouped by receiver, x of each sender gathered).  Sender pass:
// grad_x[j] of sender j (edges grouped by sender through t_perm, grad_out of
// each receiver gathered).  Each output row chunk is written once (zeros for
// a node without edges); no atomics.
// GEOM: Y holds the edge vectors r [E][3]; r_len unused
template <class S, int U, int NB, int NH, int NW, bool SEND, bool GEOM = false>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2)))
    k_radial_node(int n_nodes, const int32_t* __restrict__ ptr, const int32_t* __restrict__ perm,
                  const int32_t* __restrict__ other, const float* __restrict__ feat,
                  const float* __restrict__ Y, const float* __restrict__ r_len, RadialParams rp,
                  float* __restrict__ outp, const int32_t* __restrict__ order) {
  static_assert(U % 16 == 0 && NH % 16 == 0 && NH <= 64, "radial tiling");
  using L = W2Slice<S, NH>;
  constexpr int NA = SEND ? S::XC : S::OC;          // accumulated components per channel
  __shared__ __attribute__((aligned(16))) float w2s[L::FLOATS];
  const int c = blockIdx.y;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int e16 = lane & 15, g = lane >> 4;
  const int u = 16 * c + e16;
  float w1a[NH / 16][NB / 4];
  load_w1a<NB, NH>(rp, e16, g, w1a);
  stage_w2<S, U, NH, NW>(w2s, rp.W2, c, wv, lane);
  wait_vmcnt<0>();
  __syncthreads();
  float acc[NA];
#pragma unroll
  for (int o = 0; o < NA; ++o) acc[o] = 0.f;
  // this lane group's cursor: position pos of the launch order, its node,
  // next edge, end of the node's edges
  const int gstride = gridDim.x * NW * 4;
  int pos = (blockIdx.x * NW + wv) * 4 + g, node = 0, q = 0, qend = 0;
  auto store = [&]() {                              // the group's node row, this channel
    if constexpr (SEND) {
      float* row = outp + (size_t)node * (U * S::XC);
      static_for<S::NIN>([&](auto I) {
        constexpr int d = 2 * S::ls.v[I] + 1;
        constexpr int xo = S::xoff(I);
        static_for<d>([&](auto A) { row[U * xo + u * d + A] = acc[xo + A]; });
      });
    } else {
      float* row = outp + (size_t)node * (U * S::OC);
      static_for<S::NO>([&](auto K) {
        constexpr OutInfo oi = S::outs.o[K];
        constexpr int d = 2 * oi.l + 1;
        static_for<d>([&](auto C2) { row[U * oi.ko + u * d + C2] = acc[oi.ko + C2]; });
      });
    }
  };
  auto seek = [&]() {                               // next node with edges; zero rows on the way
    while (pos < n_nodes) {
      node = order ? min(max(order[pos], 0), n_nodes - 1) : pos;
      q = ptr[node];
      qend = ptr[node + 1];
      if (q < qend) break;
      store();                                      // acc is zero here
      pos += gstride;
    }
  };
  seek();
  // all groups of the wave step together until every one has run out of nodes
  while (__ballot(pos < n_nodes) != 0ull) {
    const bool act = pos < n_nodes;
    // gathered operands of the lane's four edges, requested first so that
    // they arrive while the hidden layer and the weights are computed; a slot
    // past the node's edges (or of a group without a node) reads a valid edge
    // and gets zero weights
    constexpr int NF = SEND ? S::OC : S::XC;
    float fr[4][NF], yr[4][S::YC];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int qq = q + r;
      const int qc = act ? (qq < qend ? qq : qend - 1) : 0;
      const int e = SEND ? perm[qc] : qc;
      radial_edge_y<S, GEOM>(Y, e, yr[r]);
      if constexpr (SEND) load_o_channel<S, U>(feat, other[qc], u, fr[r]);
      else load_x_channel<S, U>(feat, other[qc], u, fr[r]);
    }
    __builtin_amdgcn_sched_barrier(0);              // keep the loads ahead of the MFMAs
    // hidden values of tile row e16: edge e16 % 4 of group e16 / 4's node
    const int owner = 16 * (e16 >> 2);
    const int qa = __shfl(q, owner, 64) + (e16 & 3);
    const bool va = __shfl(act ? qend : 0, owner, 64) > qa;
    const int qac = va ? qa : 0;
    float bq[NB / 4], hB[NH / 4], ds[NH / 4];
    hidden_T<NB, NH>(radial_edge_len<GEOM>(Y, r_len, SEND ? perm[qac] : qac), va, rp, w1a, g, bq, hB, ds);
    f32x4 C[S::NP];
#pragma unroll
    for (int p = 0; p < S::NP; ++p) {
      C[p] = f32x4{0.f, 0.f, 0.f, 0.f};
      const float* wb = w2s + p * 16 + e16;
#pragma unroll
      for (int k = 0; k < NH / 4; ++k) C[p] = mfma_16x16x4(hB[k], wb[hid_T(k, g) * L::WS], C[p]);
    }
    static_for<4>([&](auto R) {
      float wr[S::NP];
#pragma unroll
      for (int p = 0; p < S::NP; ++p) wr[p] = C[p][int(R)];
      if constexpr (SEND) edge_bwd_send<S>(yr[R], wr, fr[R], acc);
      else edge_fwd<S>(fr[R], yr[R], wr, acc);
      __builtin_amdgcn_sched_barrier(0);          // one edge's products live at a time
    });
    if (act) {
      q += 4;
      if (q >= qend) {                              // the node is done: its row, then the next node
        store();
#pragma unroll
        for (int o = 0; o < NA; ++o) acc[o] = 0.f;
        pos += gstride;
        seek();
      }
    }
  }
}

}  // namespace tpc
