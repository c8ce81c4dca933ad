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

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma_16x16x4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

struct RadialParams {
  float r_cut;
  const float* W1;   // [NB][NH]
  const float* W2;   // [NH][P*U]
};

// Bessel basis of one length (n = 1..NB)
template <int NB>
__device__ __forceinline__ void bessel(float r, float r_cut, float (&b)[NB]) {
  const float pre = sqrtf(2.0f / r_cut) / r;
  const float k = 3.14159265358979323846f / r_cut;
#pragma unroll
  for (int n = 0; n < NB; ++n) b[n] = pre * sinf((float)(n + 1) * k * r);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// pre-activation of hidden unit hid for basis values b
template <int NB, int NH>
__device__ __forceinline__ float hidden_pre(const float (&b)[NB], const float* __restrict__ W1, int hid) {
  float s = 0.f;
#pragma unroll
  for (int n = 0; n < NB; ++n) s = fmaf(b[n], W1[n * NH + hid], s);
  return s;
}

// Per-lane A operands of the M-tile whose edge l%16 has length r (valid):
// a[k] = h[edge][4k + l/16], k = 0..NH/4-1; zero for an invalid edge.
template <int NB, int NH>
__device__ __forceinline__ void hidden_A(float r, bool valid, const RadialParams& rp, int lane,
                                         float (&a)[NH / 4]) {
  float b[NB];
  bessel<NB>(valid ? r : 1.0f, rp.r_cut, b);
#pragma unroll
  for (int k = 0; k < NH / 4; ++k) {
    const float h = silu(hidden_pre<NB, NH>(b, rp.W1, 4 * k + (lane >> 4)));
    a[k] = valid ? h : 0.f;
  }
}

// w of MT M-tiles for the 16 channels of chunk c: C[mt][p] (4 edges each)
template <class S, int U, int NH, int MT>
__device__ __forceinline__ void radial_weights(const float (&a)[MT][NH / 4], const float* __restrict__ W2,
                                               int chunk, int lane, f32x4 (&C)[MT][S::NP]) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int p = 0; p < S::NP; ++p) C[mt][p] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float* w2 = W2 + 16 * chunk + (lane & 15);
#pragma unroll 2
  for (int k = 0; k < NH / 4; ++k) {
    const float* row = w2 + (size_t)(4 * k + (lane >> 4)) * (S::NP * U);
    float b[S::NP];
#pragma unroll
    for (int p = 0; p < S::NP; ++p) b[p] = row[p * U];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int p = 0; p < S::NP; ++p) C[mt][p] = mfma_16x16x4(a[mt][k], b[p], C[mt][p]);
  }
}

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

// sum over the four lanes that share l%16 (lanes l, l^16, l^32, l^48)
template <int N>
__device__ __forceinline__ void reduce_quads(float (&v)[N]) {
#pragma unroll
  for (int t = 0; t < N; ++t) {
    v[t] += __shfl_xor(v[t], 16, 64);
    v[t] += __shfl_xor(v[t], 32, 64);
  }
}

constexpr int kRadialMT = 2;   // M-tiles (of 16 edges) per group

// ---------------------------------------------------------------------------
// forward: one wave per receiver; for each chunk of 16 channels, the weights
// of up to 32 edges at a time come from MFMA and feed the tensor product.
template <class S, int U, int NB, int NH>
__global__ void __launch_bounds__(64)
    k_radial_fwd(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col,
                 const float* __restrict__ x, const float* __restrict__ Y,
                 const float* __restrict__ r_len, RadialParams rp, float* __restrict__ out) {
  static_assert(U % 16 == 0 && NH % 4 == 0, "radial tiling");
  constexpr int MT = kRadialMT, G = 16 * MT;
  const int i = blockIdx.x;
  const int lane = threadIdx.x;
  const int beg = row_ptr[i], end = row_ptr[i + 1];
  const int ngroups = (end - beg + G - 1) / G;
  float a[MT][NH / 4];
  auto hidden = [&](int g) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int q = beg + g * G + 16 * mt + (lane & 15);
      const bool v = q < end;
      hidden_A<NB, NH>(r_len[v ? q : end - 1], v, rp, lane, a[mt]);   // end > beg here
    }
  };
  if (ngroups == 1) hidden(0);
  for (int c = 0; c < U / 16; ++c) {
    const int u = 16 * c + (lane & 15);
    float acc[S::OC];
#pragma unroll
    for (int o = 0; o < S::OC; ++o) acc[o] = 0.f;
    for (int g = 0; g < ngroups; ++g) {
      if (ngroups > 1) hidden(g);
      f32x4 C[MT][S::NP];
      radial_weights<S, U, NH, MT>(a, rp.W2, c, lane, C);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int q = beg + g * G + 16 * mt + 4 * (lane >> 4) + r;
          const int qc = q < end ? q : end - 1;   // weights of a padded edge are zero
          float xr[S::XC], yr[S::YC], wr[S::NP];
          load_x_channel<S, U>(x, col[qc], u, xr);
#pragma unroll
          for (int b = 0; b < S::YC; ++b) yr[b] = Y[(size_t)qc * S::YC + b];
#pragma unroll
          for (int p = 0; p < S::NP; ++p) wr[p] = C[mt][p][r];
          edge_fwd<S>(xr, yr, wr, acc);
        }
    }
    reduce_quads<S::OC>(acc);
    if (lane < 16) {
      float* row = out + (size_t)i * (U * S::OC);
      static_for<S::NO>([&](auto K) {
        constexpr OutInfo oi = S::outs.o[K];
        constexpr int d = 2 * oi.l + 1;
        static_for<d>([&](auto C2) { row[U * oi.ko + u * d + C2] = acc[oi.ko + C2]; });
      });
    }
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

// hidden values (B operands of the transposed tile) and SiLU derivatives of the
// lane's edge; both zero for an invalid edge
template <int NB, int NH>
__device__ __forceinline__ void hidden_T(float r, bool valid, const RadialParams& rp, int g,
                                         float (&b)[NB], float (&hB)[NH / 4], float (&ds)[NH / 4]) {
  bessel<NB>(valid ? r : 1.0f, rp.r_cut, b);
#pragma unroll
  for (int k = 0; k < NH / 4; ++k) {
    const float z = hidden_pre<NB, NH>(b, rp.W1, hid_T(k, g));
    const float s = 1.0f / (1.0f + expf(-z));
    hB[k] = valid ? z * s : 0.f;
    ds[k] = valid ? s * (1.0f + z * (1.0f - s)) : 0.f;
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

template <class S, int U>
__device__ __forceinline__ void load_o4(const float* __restrict__ g, int i, int u0, float (&gr)[4][S::OC]) {
  const float* row = g + (size_t)i * (U * S::OC);
  static_for<S::NO>([&](auto K) {
    constexpr OutInfo oi = S::outs.o[K];
    constexpr int d = 2 * oi.l + 1;
    const float4* p = reinterpret_cast<const float4*>(row + U * oi.ko + u0 * d);
    float v[4 * d];
    static_for<d>([&](auto Q) {
      const float4 t = p[Q];
      v[4 * Q + 0] = t.x; v[4 * Q + 1] = t.y; v[4 * Q + 2] = t.z; v[4 * Q + 3] = t.w;
    });
    static_for<4>([&](auto I2) { static_for<d>([&](auto C) { gr[I2][oi.ko + C] = v[I2 * d + C]; }); });
  });
}

// Receiver pass: one wave walks receivers i = blockIdx.x, +gridDim.x, ...; per
// 16-edge tile and chunk of 16 channels, each path p gives w (MFMA), the Z-form
// adjoint (grad_w_p, grad_Y += w_p Z_p) and grad_h += W2_p grad_w_p (MFMA).
// grad_W1 = B^T (grad_h * SiLU') is reduced through LDS into one partial per
// workgroup (part[blockIdx.x][n][hid]), summed later in a fixed order.
template <class S, int U, int NB, int NH>
__global__ void __launch_bounds__(64)
    k_radial_bwd_recv(int n_nodes, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col,
                      const float* __restrict__ x, const float* __restrict__ Y,
                      const float* __restrict__ r_len, RadialParams rp, const float* __restrict__ gout,
                      float* __restrict__ grad_Y, float* __restrict__ part) {
  static_assert(U % 16 == 0 && NH % 16 == 0 && NH <= 64, "radial tiling");
  constexpr int LD = S::NP * U;      // row length of W2
  __shared__ float s_gp[16][NH + 1];
  __shared__ float s_b[16][NB];
  const int lane = threadIdx.x, e16 = lane & 15, g = lane >> 4;
  float w1[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) w1[n] = 0.f;
  for (int i = blockIdx.x; i < n_nodes; i += gridDim.x) {
    const int beg = row_ptr[i], end = row_ptr[i + 1];
    for (int t0 = beg; t0 < end; t0 += 16) {
      const int q = t0 + e16;
      const bool valid = q < end;
      const int qc = valid ? q : end - 1;
      const int j = col[qc];
      float b[NB], hB[NH / 4], ds[NH / 4], yr[S::YC], gy[S::YC];
      hidden_T<NB, NH>(r_len[qc], valid, rp, g, b, hB, ds);
#pragma unroll
      for (int t = 0; t < S::YC; ++t) {
        yr[t] = Y[(size_t)qc * S::YC + t];
        gy[t] = 0.f;
      }
      f32x4 gh[NH / 16];
#pragma unroll
      for (int t = 0; t < NH / 16; ++t) gh[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
      for (int c = 0; c < U / 16; ++c) {
        const int u0 = 16 * c + 4 * g;
        float xr[4][S::XC], gr[4][S::OC];
        load_x4<S, U>(x, j, u0, xr);
        load_o4<S, U>(gout, i, u0, gr);
        static_for<S::NP>([&](auto P) {
          constexpr PathInfo pi = S::paths.p[P];
          using T = CgPath<pi.l1, pi.l2, pi.l3>;
          constexpr int D2 = 2 * pi.l2 + 1;
          // w[channel 16c + 4g + r][edge e16], r = 0..3
          const float* wa = rp.W2 + P * U + 16 * c + e16;
          f32x4 w = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int k = 0; k < NH / 4; ++k) w = mfma_16x16x4(wa[(size_t)hid_T(k, g) * LD], hB[k], w);
          float gw[4];
          static_for<4>([&](auto R) {
            float z[D2];
            static_for<D2>([&](auto B2) { z[B2] = 0.f; });
            static_for<T::nnz>([&](auto N) {
              constexpr Nz e = T::table.e[N];
              z[e.b] = fmaf(e.v, xr[R][pi.xo + e.a] * gr[R][pi.ko + e.c], z[e.b]);
            });
            float s = 0.f;
            static_for<D2>([&](auto B2) {
              s = fmaf(yr[pi.yo + B2], z[B2], s);
              gy[pi.yo + B2] = fmaf(w[int(R)], z[B2], gy[pi.yo + B2]);
            });
            gw[R] = s;
          });
          // grad_h[hid 16t + 4g + r][edge e16] += sum over the chunk's channels
          const float* wb = rp.W2 + (size_t)e16 * LD + P * U + u0;
#pragma unroll
          for (int t = 0; t < NH / 16; ++t) {
            const float4 a4 = *reinterpret_cast<const float4*>(wb + (size_t)16 * t * LD);
            gh[t] = mfma_16x16x4(a4.x, gw[0], gh[t]);
            gh[t] = mfma_16x16x4(a4.y, gw[1], gh[t]);
            gh[t] = mfma_16x16x4(a4.z, gw[2], gh[t]);
            gh[t] = mfma_16x16x4(a4.w, gw[3], gh[t]);
          }
        });
      }
      // grad_Y: sum over the four channel groups of the edge
#pragma unroll
      for (int t = 0; t < S::YC; ++t) {
        gy[t] += __shfl_xor(gy[t], 16, 64);
        gy[t] += __shfl_xor(gy[t], 32, 64);
      }
      if (grad_Y && g == 0 && valid) {
#pragma unroll
        for (int t = 0; t < S::YC; ++t) grad_Y[(size_t)q * S::YC + t] = gy[t];
      }
      // grad_W1[n][hid] += sum over the tile's edges of B_n * grad_pre[hid]
#pragma unroll
      for (int k = 0; k < NH / 4; ++k) s_gp[e16][hid_T(k, g)] = gh[k >> 2][k & 3] * ds[k];
      if (g == 0) {
#pragma unroll
        for (int n = 0; n < NB; ++n) s_b[e16][n] = b[n];
      }
      __syncthreads();
      if (lane < NH) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float gp = s_gp[e][lane];
#pragma unroll
          for (int n = 0; n < NB; ++n) w1[n] = fmaf(s_b[e][n], gp, w1[n]);
        }
      }
      __syncthreads();
    }
  }
  if (lane < NH) {
    float* p = part + (size_t)blockIdx.x * (NB * NH);
#pragma unroll
    for (int n = 0; n < NB; ++n) p[n * NH + lane] = w1[n];
  }
}

// grad_W2 pass: workgroup (block, chunk c) with one wave per group of PGS
// paths; the waves walk the same receivers' edges.  Tile: M = 16 hidden units,
// N = 16 channels, K = edges; lane l owns channel 16c + l%16 and edges
// 4(l/16)..+3 of a 16-edge tile.  The hidden values come from a small MFMA
// (pre = B W1, K = NB) whose D layout is exactly the A operand needed here.
template <class S, int U, int NB, int NH, int PGS>
__global__ void __launch_bounds__(64 * ((S::NP + PGS - 1) / PGS))
    k_radial_bwd_w2(int n_nodes, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col,
                    const float* __restrict__ x, const float* __restrict__ Y,
                    const float* __restrict__ r_len, RadialParams rp, const float* __restrict__ gout,
                    float* __restrict__ part) {
  static_assert(U % 16 == 0 && NH % 16 == 0 && NB % 4 == 0, "radial tiling");
  constexpr int NPG = (S::NP + PGS - 1) / PGS;
  constexpr int LD = S::NP * U;
  const int c = blockIdx.y;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int e16 = lane & 15, g = lane >> 4;
  const int u = 16 * c + e16;
  static_for<NPG>([&](auto G) {
    if (wv != G) return;
    constexpr int P0 = G * PGS;
    constexpr int NPP = S::NP - P0 < PGS ? S::NP - P0 : PGS;
    f32x4 acc[NPP][NH / 16];
    static_for<NPP>([&](auto PP) {
#pragma unroll
      for (int t = 0; t < NH / 16; ++t) acc[PP][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    });
    for (int i = blockIdx.x; i < n_nodes; i += gridDim.x) {
      const int beg = row_ptr[i], end = row_ptr[i + 1];
      if (beg == end) continue;
      float gr[S::OC];
      load_o_channel<S, U>(gout, i, u, gr);
      for (int t0 = beg; t0 < end; t0 += 16) {
        // pre[edge 4g + r][hid 16t + e16] via MFMA: A = B_n(edge e16), B = W1
        const int qa = t0 + e16;
        const bool va = qa < end;
        const float ra = va ? r_len[qa < end ? qa : end - 1] : 1.0f;
        const float pre_b = sqrtf(2.0f / rp.r_cut) / ra;
        const float kk = 3.14159265358979323846f / rp.r_cut;
        float bn[NB / 4];
#pragma unroll
        for (int s = 0; s < NB / 4; ++s)
          bn[s] = va ? pre_b * sinf((float)(4 * s + g + 1) * kk * ra) : 0.f;
        float hA[NH / 16][4];
#pragma unroll
        for (int t = 0; t < NH / 16; ++t) {
          f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < NB / 4; ++s) z = mfma_16x16x4(bn[s], rp.W1[(4 * s + g) * NH + 16 * t + e16], z);
#pragma unroll
          for (int r = 0; r < 4; ++r) hA[t][r] = silu(z[r]);
        }
        // grad_w of this wave's paths for the lane's four edges
        float gw[NPP][4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int q = t0 + 4 * g + r;
          const int qc = q < end ? q : end - 1;   // its hidden values are zero
          float xr[S::XC], yr[S::YC];
          load_x_channel<S, U>(x, col[qc], u, xr);
#pragma unroll
          for (int t = 0; t < S::YC; ++t) yr[t] = Y[(size_t)qc * S::YC + t];
          static_for<NPP>([&](auto PP) {
            constexpr PathInfo pi = S::paths.p[P0 + PP];
            using T = CgPath<pi.l1, pi.l2, pi.l3>;
            constexpr int D2 = 2 * pi.l2 + 1;
            float z[D2];
            static_for<D2>([&](auto B2) { z[B2] = 0.f; });
            static_for<T::nnz>([&](auto N) {
              constexpr Nz e = T::table.e[N];
              z[e.b] = fmaf(e.v, xr[pi.xo + e.a] * gr[pi.ko + e.c], z[e.b]);
            });
            float s = 0.f;
            static_for<D2>([&](auto B2) { s = fmaf(yr[pi.yo + B2], z[B2], s); });
            gw[PP][r] = s;
          });
        }
        static_for<NPP>([&](auto PP) {
#pragma unroll
          for (int t = 0; t < NH / 16; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[PP][t] = mfma_16x16x4(hA[t][r], gw[PP][r], acc[PP][t]);
        });
      }
    }
    // part[block][hid][p*U + u] (each chunk writes its own columns)
    float* pb = part + (size_t)blockIdx.x * NH * LD;
    static_for<NPP>([&](auto PP) {
#pragma unroll
      for (int t = 0; t < NH / 16; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) pb[(size_t)(16 * t + 4 * g + r) * LD + (P0 + PP) * U + u] = acc[PP][t][r];
    });
  });
}

// Sender pass (grad_x): the forward's structure over the sender grouping; w is
// recomputed per chunk by MFMA, grad_out of each edge's receiver is gathered.
template <class S, int U, int NB, int NH>
__global__ void __launch_bounds__(64)
    k_radial_bwd_send(const int32_t* __restrict__ t_row_ptr, const int32_t* __restrict__ t_perm,
                      const int32_t* __restrict__ t_col, const float* __restrict__ Y,
                      const float* __restrict__ r_len, RadialParams rp, const float* __restrict__ gout,
                      float* __restrict__ grad_x) {
  static_assert(U % 16 == 0 && NH % 4 == 0, "radial tiling");
  constexpr int MT = kRadialMT, G = 16 * MT;
  const int j = blockIdx.x;
  const int lane = threadIdx.x;
  const int beg = t_row_ptr[j], end = t_row_ptr[j + 1];
  const int ngroups = (end - beg + G - 1) / G;
  float a[MT][NH / 4];
  auto hidden = [&](int gi) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int q = beg + gi * G + 16 * mt + (lane & 15);
      const bool v = q < end;
      hidden_A<NB, NH>(r_len[t_perm[v ? q : end - 1]], v, rp, lane, a[mt]);   // end > beg here
    }
  };
  if (ngroups == 1) hidden(0);
  for (int c = 0; c < U / 16; ++c) {
    const int u = 16 * c + (lane & 15);
    float acc[S::XC];
#pragma unroll
    for (int o = 0; o < S::XC; ++o) acc[o] = 0.f;
    for (int gi = 0; gi < ngroups; ++gi) {
      if (ngroups > 1) hidden(gi);
      f32x4 C[MT][S::NP];
      radial_weights<S, U, NH, MT>(a, rp.W2, c, lane, C);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int q = beg + gi * G + 16 * mt + 4 * (lane >> 4) + r;
          const int qc = q < end ? q : end - 1;   // weights of a padded edge are zero
          const int e = t_perm[qc];
          float gr[S::OC], yr[S::YC], wr[S::NP];
          load_o_channel<S, U>(gout, t_col[qc], u, gr);
#pragma unroll
          for (int b = 0; b < S::YC; ++b) yr[b] = Y[(size_t)e * S::YC + b];
#pragma unroll
          for (int p = 0; p < S::NP; ++p) wr[p] = C[mt][p][r];
          edge_bwd_send<S>(yr, wr, gr, acc);
        }
    }
    reduce_quads<S::XC>(acc);
    if (lane < 16) {
      float* row = grad_x + (size_t)j * (U * S::XC);
      static_for<S::NIN>([&](auto I) {
        constexpr int d = 2 * S::ls.v[I] + 1;
        constexpr int xo = S::xoff(I);
        static_for<d>([&](auto A) { row[U * xo + u * d + A] = acc[xo + A]; });
      });
    }
  }
}

}  // namespace tpc
