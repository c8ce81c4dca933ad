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
      hidden_A<NB, NH>(v ? r_len[q] : 1.f, v, rp, lane, a[mt]);
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

}  // namespace tpc
