// Second-order backward of the radial-weight convolution: the gradients of
// L = <gg_x, grad_x> + <gg_Y, grad_Y> + <gg_r, grad_rlen> (cotangents on the
// first backward's outputs that a loss on forces produces) with respect to
// x, Y, r_len, W1, W2 and the unmixed upstream gradient g, with the radial
// weights recomputed on chip as in the first-order passes ("Sobek: Streaming
// Equivariant Tensor Product Convolutions", Abstract: forward, backward and
// double backward with the radial projection streamed).
//
// With F(g, x, Y, w) = <g, out(x, Y, w)> and v = gg_r dw/dr (the weights'
// tangent along gg_r),
//   L = F(g, gg_x, Y, w) + F(g, x, gg_Y, w) + F(g, x, Y, v),
// so every pass is a first-order pass with more operands:
//   k_radial_node_dbl<false>  out_dot = out(gg_x, Y, w) + out(x, gg_Y, w) + out(x, Y, v)
//                             (d_g before the mix), receiver-grouped;
//   k_radial_node_dbl<true>   d_x = gx(gg_Y, w, g) + gx(Y, v, g), sender-grouped;
//   k_radial_dbl_recv         d_Y = gY(gg_x, w, g) + gY(x, v, g) and, from the
//                             weights' cotangent dw = gw(gg_x, Y, g) + gw(x, gg_Y, g)
//                             and the tangent's dv = gw(x, Y, g), the chain rule
//                             through pre = B W1, h = SiLU(pre), a = B' W1,
//                             t = SiLU'(pre) a: d_pre = SiLU' dh + SiLU'' a dt,
//                             d_a = SiLU' dt (dh = W2 dw, dt = gg_r W2 dv), giving
//                             d_W1 = B^T d_pre + B'^T d_a and
//                             d_rlen = B' . (W1 d_pre) + B'' . (W1 d_a);
//   k_radial_dbl_w2<KIND>     d_W2 = h^T dw + (gg_r t)^T dv, one launch per term.
// The tile layouts, W2 staging and fixed-order partial sums are those of the
// first-order kernels.  A missing cotangent pointer reads as zeros.
#pragma once
#include "radial_kernels.hpp"

namespace tpc {

// The lane's edge (edge l%16 of a 16-edge tile) in the K-slot order of
// hidden_T: basis values bq[s] = B_{4s+g+1}(r) and derivatives bd[s] =
// B'_{4s+g+1}(r), the pre-activations pre[k] and their derivative in r,
// ap[k] = (B' W1)[hid_T(k, g)], both from the small MFMA.  All zero for an
// invalid edge.
template <int NB, int NH>
__device__ __forceinline__ void hidden_jet(float r, bool valid, const RadialParams& rp,
                                           const float (&w1a)[NH / 16][NB / 4], int g, float (&bq)[NB / 4],
                                           float (&bd)[NB / 4], float (&pre)[NH / 4], float (&ap)[NH / 4]) {
  static_assert(NB % 4 == 0 && NH % 16 == 0, "hidden tiling");
  const float rr = valid ? r : 1.0f;
  const float c = sqrtf(2.0f / rp.r_cut);
  const float inv = 1.0f / rr;
  const float kk = 3.14159265358979323846f / rp.r_cut;
#pragma unroll
  for (int s = 0; s < NB / 4; ++s) {
    const float kn = (float)(4 * s + g + 1) * kk;
    const float sn = sinf(kn * rr), cs = cosf(kn * rr);
    bq[s] = valid ? c * sn * inv : 0.f;
    bd[s] = valid ? c * (kn * cs * inv - sn * inv * inv) : 0.f;
  }
#pragma unroll
  for (int t = 0; t < NH / 16; ++t) {
    f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f}, za = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NB / 4; ++s) {
      z = mfma_16x16x4(w1a[t][s], bq[s], z);
      za = mfma_16x16x4(w1a[t][s], bd[s], za);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pre[4 * t + i] = z[i];
      ap[4 * t + i] = za[i];
    }
  }
}

// SiLU and its first two derivatives from the logistic function sg = sigma(z)
__device__ __forceinline__ float silu_d1(float z, float sg) { return sg * (1.0f + z * (1.0f - sg)); }
__device__ __forceinline__ float silu_d2(float z, float sg) {
  return sg * (1.0f - sg) * (2.0f + z * (1.0f - 2.0f * sg));
}

// hB = SiLU(pre) and tB = gg_r SiLU'(pre) a (the tangent of the hidden values
// along gg_r), zero for an invalid edge
template <int NH>
__device__ __forceinline__ void hidden_tangent(bool valid, float ggr, const float (&pre)[NH / 4],
                                               const float (&ap)[NH / 4], float (&hB)[NH / 4],
                                               float (&tB)[NH / 4]) {
#pragma unroll
  for (int k = 0; k < NH / 4; ++k) {
    const float sg = sigmoid_fast(pre[k]);
    hB[k] = valid ? pre[k] * sg : 0.f;
    tB[k] = valid ? ggr * silu_d1(pre[k], sg) * ap[k] : 0.f;
  }
}

// Forward tangent (SEND = false) and sender pass (SEND = true) of the
// second-order backward, chunk-major as k_radial_node.  Per 16-edge tile the
// weights w (A operand hB) and their tangent v (A operand tB) come from the
// w-MFMA on the chunk's W2 slice; then, per edge of the lane:
//   SEND = false: acc += T(gg_x, Y, w) + T(x, gg_Y, w) + T(x, Y, v)
//                 (feat = x, gfeat = gg_x; output rows: out_dot)
//   SEND = true:  acc += gx(gg_Y, w, g) + gx(Y, v, g)
//                 (feat = g, the unmixed upstream gradient; output rows: d_x)
// The w terms are done before v is formed, so one set of weight registers
// serves both.
template <class S, int U, int NB, int NH, int NW, bool SEND>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2)))
    k_radial_node_dbl(int n_nodes, const int32_t* __restrict__ ptr, const int32_t* __restrict__ perm,
                      const int32_t* __restrict__ other, const float* __restrict__ feat,
                      const float* __restrict__ gfeat, const float* __restrict__ Y,
                      const float* __restrict__ ggY, const float* __restrict__ r_len,
                      const float* __restrict__ ggr, RadialParams rp, float* __restrict__ outp,
                      const int32_t* __restrict__ order) {
  static_assert(U % 16 == 0 && NH % 16 == 0 && NH <= 64, "radial tiling");
  using L = W2Slice<S, NH>;
  constexpr int NA = SEND ? S::XC : S::OC;          // accumulated components per channel
  constexpr int NF = SEND ? S::OC : S::XC;          // gathered components per channel
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
  // positions of the launch order, their nodes i
  for (int pos = blockIdx.x * NW + wv; pos < n_nodes; pos += gridDim.x * NW) {
    const int i = order ? min(max(order[pos], 0), n_nodes - 1) : pos;
    const int beg = ptr[i], end = ptr[i + 1];
    float acc[NA];
#pragma unroll
    for (int o = 0; o < NA; ++o) acc[o] = 0.f;
    for (int t0 = beg; t0 < end; t0 += 16) {
      float fr[4][NF], yr[4][S::YC];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int q = t0 + 4 * g + r;
        const int qc = q < end ? q : end - 1;       // weights of a padded edge are zero
        const int e = SEND ? perm[qc] : qc;
#pragma unroll
        for (int b = 0; b < S::YC; ++b) yr[r][b] = Y[(size_t)e * S::YC + b];
        if constexpr (SEND) load_o_channel<S, U>(feat, other[qc], u, fr[r]);
        else load_x_channel<S, U>(feat, other[qc], u, fr[r]);
      }
      __builtin_amdgcn_sched_barrier(0);
      const int qa = t0 + e16;
      const bool va = qa < end;
      const int ea = SEND ? perm[va ? qa : end - 1] : (va ? qa : end - 1);
      const float gga = (ggr && va) ? ggr[ea] : 0.f;
      float hB[NH / 4], tB[NH / 4];
      {
        float bq[NB / 4], bd[NB / 4], pre[NH / 4], ap[NH / 4];
        hidden_jet<NB, NH>(r_len[ea], va, rp, w1a, g, bq, bd, pre, ap);
        hidden_tangent<NH>(va, gga, pre, ap, hB, tB);
      }
      f32x4 C[S::NP];
      // the w terms
#pragma unroll
      for (int p = 0; p < S::NP; ++p) {
        C[p] = f32x4{0.f, 0.f, 0.f, 0.f};
        const float* wb = w2s + p * 16 + e16;
#pragma unroll
        for (int k = 0; k < NH / 4; ++k) C[p] = mfma_16x16x4(hB[k], wb[hid_T(k, g) * L::WS], C[p]);
      }
      static_for<4>([&](auto R) {
        const int q = t0 + 4 * g + R;
        const int qc = q < end ? q : end - 1;
        const int e = SEND ? perm[qc] : qc;
        float wr[S::NP];
#pragma unroll
        for (int p = 0; p < S::NP; ++p) wr[p] = C[p][int(R)];
        if constexpr (SEND) {
          if (ggY) {
            float gy[S::YC];
#pragma unroll
            for (int b = 0; b < S::YC; ++b) gy[b] = ggY[(size_t)e * S::YC + b];
            edge_bwd_send<S>(gy, wr, fr[R], acc);
          }
        } else {
          if (gfeat) {
            float gx[S::XC];
            load_x_channel<S, U>(gfeat, other[qc], u, gx);
            edge_fwd<S>(gx, yr[R], wr, acc);
          }
          if (ggY) {
            float gy[S::YC];
#pragma unroll
            for (int b = 0; b < S::YC; ++b) gy[b] = ggY[(size_t)e * S::YC + b];
            edge_fwd<S>(fr[R], gy, wr, acc);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      // the tangent term
      if (ggr) {
#pragma unroll
        for (int p = 0; p < S::NP; ++p) {
          C[p] = f32x4{0.f, 0.f, 0.f, 0.f};
          const float* wb = w2s + p * 16 + e16;
#pragma unroll
          for (int k = 0; k < NH / 4; ++k) C[p] = mfma_16x16x4(tB[k], wb[hid_T(k, g) * L::WS], C[p]);
        }
        static_for<4>([&](auto R) {
          float vr[S::NP];
#pragma unroll
          for (int p = 0; p < S::NP; ++p) vr[p] = C[p][int(R)];
          if constexpr (SEND) edge_bwd_send<S>(yr[R], vr, fr[R], acc);
          else edge_fwd<S>(fr[R], yr[R], vr, acc);
          __builtin_amdgcn_sched_barrier(0);
        });
      }
    }
    reduce_quads<NA>(acc);
    if (lane < 16) {
      if constexpr (SEND) {
        float* row = outp + (size_t)i * (U * S::XC);
        static_for<S::NIN>([&](auto I) {
          constexpr int d = 2 * S::ls.v[I] + 1;
          constexpr int xo = S::xoff(I);
          static_for<d>([&](auto A) { row[U * xo + u * d + A] = acc[xo + A]; });
        });
      } else {
        float* row = outp + (size_t)i * (U * S::OC);
        static_for<S::NO>([&](auto K) {
          constexpr OutInfo oi = S::outs.o[K];
          constexpr int d = 2 * oi.l + 1;
          static_for<d>([&](auto C2) { row[U * oi.ko + u * d + C2] = acc[oi.ko + C2]; });
        });
      }
    }
  }
}

// Receiver pass of the second-order backward (tile transposed as in
// k_radial_bwd_recv: lane l owns edge l%16 and channels 4(l/16)..+3 of the
// chunk).  Per chunk and path: w and v (MFMA, B operands hB and tB), the
// Z-forms of x and gg_x against g,
//   Zx[b] = sum_{a,c} C x_a g_c,   Zg[b] = sum_{a,c} C gg_x_a g_c,
// then d_Y[b] += w Zg[b] + v Zx[b], dw = sum_b Y_b Zg[b] + gg_Y_b Zx[b],
// dv = sum_b Y_b Zx[b], and dh += W2 dw, dt += W2 dv (MFMA).  The terms of
// x and those of gg_x run one after the other, so the two node rows are not
// in registers at the same time.  After the
// chunks: d_Y summed over the edge's channel lanes and stored; d_pre and d_a
// from the SiLU derivatives; d_rlen from W1 d_pre and W1 d_a (MFMA) against
// B' and B''; d_W1 partial per wave through LDS.
template <class S, int U, int NB, int NH, int NW>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1, 1)))
    k_radial_dbl_recv(int n_nodes, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col,
                      const float* __restrict__ x, const float* __restrict__ ggx, const float* __restrict__ Y,
                      const float* __restrict__ ggY, const float* __restrict__ r_len,
                      const float* __restrict__ ggr, RadialParams rp, const float* __restrict__ gout,
                      float* __restrict__ d_Y, float* __restrict__ d_rlen, float* __restrict__ part,
                      const int32_t* __restrict__ order) {
  static_assert(U % 16 == 0 && NH % 16 == 0 && NH <= 64 && NB <= 16, "radial tiling");
  using L = W2Slice<S, NH>;
  constexpr int GF = 16 * S::OC;                    // staged upstream-gradient floats per wave
  constexpr int HS = NH + 1;
  constexpr int RED = 2 * 16 * HS + 2 * 16 * NB;    // d_W1 scratch floats per wave
  static_assert(NW * RED <= L::FLOATS, "d_W1 scratch reuses the W2 slice");
  __shared__ __attribute__((aligned(16))) float smem[L::FLOATS + NW * GF];
  float* w2s = smem;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int e16 = lane & 15, g = lane >> 4;
  float* gs = smem + L::FLOATS + wv * GF;
  float* red = smem + wv * RED;
  float w1a[NH / 16][NB / 4];
  load_w1a<NB, NH>(rp, e16, g, w1a);
  float w1[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) w1[n] = 0.f;
  const int stride = gridDim.x * NW;
  int pos = blockIdx.x * NW + wv, i = 0, t0 = 0, end = 0;   // position of the launch order, its node
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
  while (__syncthreads_or(pos < n_nodes)) {
    const bool has = pos < n_nodes;
    const int q = t0 + e16;
    const bool valid = has && q < end;
    const int qc = has ? (q < end ? q : end - 1) : 0;
    const int j = has ? col[qc] : 0;
    const float rl = has ? r_len[qc] : 1.f;
    const float gg = (ggr && valid) ? ggr[qc] : 0.f;
    float hB[NH / 4], tB[NH / 4];
    {
      float bq0[NB / 4], bd0[NB / 4], pre0[NH / 4], ap0[NH / 4];   // recomputed after the chunks
      hidden_jet<NB, NH>(rl, valid, rp, w1a, g, bq0, bd0, pre0, ap0);
      hidden_tangent<NH>(valid, gg, pre0, ap0, hB, tB);
    }
    float yr[S::YC], gyr[S::YC], dy[S::YC];
#pragma unroll
    for (int t = 0; t < S::YC; ++t) {
      yr[t] = has ? Y[(size_t)qc * S::YC + t] : 0.f;
      gyr[t] = (has && ggY) ? ggY[(size_t)qc * S::YC + t] : 0.f;
      dy[t] = 0.f;
    }
    f32x4 gh[NH / 16], gt[NH / 16];
#pragma unroll
    for (int t = 0; t < NH / 16; ++t) {
      gh[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      gt[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
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
        // phase 1, the Z-form of x: dv = sum_b Y_b Zx[b], the gg_Y part of dw,
        // d_Y += v Zx
        static_for<S::NP>([&](auto P) {
          constexpr PathInfo pi = S::paths.p[P];
          using T = CgPath<pi.l1, pi.l2, pi.l3>;
          constexpr int D2 = 2 * pi.l2 + 1, D3 = 2 * pi.l3 + 1;
          const float* wa = w2s + P * 16 + e16;
          f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int k = 0; k < NH / 4; ++k) v = mfma_16x16x4(wa[hid_T(k, g) * L::WS], tB[k], v);
          float gb[4 * D3];
          const float4* gp = reinterpret_cast<const float4*>(gs + 16 * pi.ko + 4 * g * D3);
          static_for<D3>([&](auto Q) {
            const float4 t = gp[Q];
            gb[4 * Q + 0] = t.x; gb[4 * Q + 1] = t.y; gb[4 * Q + 2] = t.z; gb[4 * Q + 3] = t.w;
          });
          float dw[4], dv[4];
          static_for<4>([&](auto R) {
            float zx[D2];
            zform_scaled<pi.l1, pi.l2, pi.l3, pi.xo, R * D3>(xr[R], gb, zx);
            float sw = 0.f, sv = 0.f;
            static_for<D2>([&](auto B2) {
              sw = fmaf(gyr[pi.yo + B2], zx[B2], sw);
              sv = fmaf(yr[pi.yo + B2], zx[B2], sv);
              dy[pi.yo + B2] = fmaf(v[int(R)], zx[B2], dy[pi.yo + B2]);
            });
            dw[R] = sw;
            dv[R] = sv;
          });
          const float* wb = w2s + e16 * L::WS + P * 16 + 4 * g;
#pragma unroll
          for (int t = 0; t < NH / 16; ++t) {
            const float4 a4 = *reinterpret_cast<const float4*>(wb + 16 * t * L::WS);
            gh[t] = mfma_16x16x4(a4.x, dw[0], gh[t]);
            gh[t] = mfma_16x16x4(a4.y, dw[1], gh[t]);
            gh[t] = mfma_16x16x4(a4.z, dw[2], gh[t]);
            gh[t] = mfma_16x16x4(a4.w, dw[3], gh[t]);
            gt[t] = mfma_16x16x4(a4.x, dv[0], gt[t]);
            gt[t] = mfma_16x16x4(a4.y, dv[1], gt[t]);
            gt[t] = mfma_16x16x4(a4.z, dv[2], gt[t]);
            gt[t] = mfma_16x16x4(a4.w, dv[3], gt[t]);
          }
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      if (ggx) {
        // phase 2, the Z-form of gg_x: the Y part of dw, d_Y += w Zg
        load_x4<S, U>(ggx, j, u0, xr);
        wait_vmcnt<0>();
        if (has) {
          static_for<S::NP>([&](auto P) {
            constexpr PathInfo pi = S::paths.p[P];
            using T = CgPath<pi.l1, pi.l2, pi.l3>;
            constexpr int D2 = 2 * pi.l2 + 1, D3 = 2 * pi.l3 + 1;
            const float* wa = w2s + P * 16 + e16;
            f32x4 w = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < NH / 4; ++k) w = mfma_16x16x4(wa[hid_T(k, g) * L::WS], hB[k], w);
            float gb[4 * D3];
            const float4* gp = reinterpret_cast<const float4*>(gs + 16 * pi.ko + 4 * g * D3);
            static_for<D3>([&](auto Q) {
              const float4 t = gp[Q];
              gb[4 * Q + 0] = t.x; gb[4 * Q + 1] = t.y; gb[4 * Q + 2] = t.z; gb[4 * Q + 3] = t.w;
            });
            float dw[4];
            static_for<4>([&](auto R) {
              float zg[D2];
              zform_scaled<pi.l1, pi.l2, pi.l3, pi.xo, R * D3>(xr[R], gb, zg);
              float sw = 0.f;
              static_for<D2>([&](auto B2) {
                sw = fmaf(yr[pi.yo + B2], zg[B2], sw);
                dy[pi.yo + B2] = fmaf(w[int(R)], zg[B2], dy[pi.yo + B2]);
              });
              dw[R] = sw;
            });
            const float* wb = w2s + e16 * L::WS + P * 16 + 4 * g;
#pragma unroll
            for (int t = 0; t < NH / 16; ++t) {
              const float4 a4 = *reinterpret_cast<const float4*>(wb + 16 * t * L::WS);
              gh[t] = mfma_16x16x4(a4.x, dw[0], gh[t]);
              gh[t] = mfma_16x16x4(a4.y, dw[1], gh[t]);
              gh[t] = mfma_16x16x4(a4.z, dw[2], gh[t]);
              gh[t] = mfma_16x16x4(a4.w, dw[3], gh[t]);
            }
            __builtin_amdgcn_sched_barrier(0);
          });
        }
      }
    }
#pragma unroll
    for (int t = 0; t < S::YC; ++t) {
      dy[t] += __shfl_xor(dy[t], 16, 64);
      dy[t] += __shfl_xor(dy[t], 32, 64);
    }
    if (d_Y && g == 0 && valid) {
#pragma unroll
      for (int t = 0; t < S::YC; ++t) d_Y[(size_t)q * S::YC + t] = dy[t];
    }
    // basis values and network derivatives again (not kept through the chunks)
    float bq[NB / 4], bd[NB / 4], dpre[NH / 4], da[NH / 4];
    {
      float rl2 = rl, pre[NH / 4], ap[NH / 4];
      asm volatile("" : "+v"(rl2));
      hidden_jet<NB, NH>(rl2, valid, rp, w1a, g, bq, bd, pre, ap);
#pragma unroll
      for (int k = 0; k < NH / 4; ++k) {
        const float sg = sigmoid_fast(pre[k]);
        const float s1 = valid ? silu_d1(pre[k], sg) : 0.f;
        const float s2 = valid ? silu_d2(pre[k], sg) : 0.f;
        const float dh = gh[k >> 2][k & 3], dt = gg * gt[k >> 2][k & 3];
        dpre[k] = s1 * dh + s2 * ap[k] * dt;
        da[k] = s1 * dt;
      }
    }
    if (d_rlen && has) {
      // (W1 d_pre)[n][edge] and (W1 d_a)[n][edge] on the MFMA (rows n >= NB
      // zero); lane l gets n = 4(l/16) + i of edge l%16
      f32x4 gB = f32x4{0.f, 0.f, 0.f, 0.f}, gA = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < NH / 4; ++k) {
        const float a = e16 < NB ? rp.W1[e16 * NH + hid_T(k, g)] : 0.f;
        gB = mfma_16x16x4(a, dpre[k], gB);
        gA = mfma_16x16x4(a, da[k], gA);
      }
      const float cb = sqrtf(2.0f / rp.r_cut), kk = 3.14159265358979323846f / rp.r_cut;
      const float inv = 1.0f / rl;
      float acc = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int n = 4 * g + t;
        if (n < NB) {
          const float kn = (float)(n + 1) * kk;
          const float sn = sinf(kn * rl), cs = cosf(kn * rl);
          const float b1 = cb * (kn * cs * inv - sn * inv * inv);
          const float b2 = cb * (-kn * kn * sn * inv - 2.0f * kn * cs * inv * inv + 2.0f * sn * inv * inv * inv);
          acc += gB[t] * b1 + gA[t] * b2;
        }
      }
      acc += __shfl_xor(acc, 16, 64);
      acc += __shfl_xor(acc, 32, 64);
      if (g == 0 && valid) d_rlen[q] = acc;
    }
    // d_W1[n][hid] += sum over the tile's edges of B_n d_pre[hid] + B'_n d_a[hid]
    __syncthreads();                                // W2 slice no longer read
    if (has) {
      float* s_dp = red;
      float* s_da = red + 16 * HS;
      float* s_b = red + 2 * 16 * HS;
      float* s_bd = s_b + 16 * NB;
#pragma unroll
      for (int k = 0; k < NH / 4; ++k) {
        s_dp[e16 * HS + hid_T(k, g)] = dpre[k];
        s_da[e16 * HS + hid_T(k, g)] = da[k];
      }
#pragma unroll
      for (int t = 0; t < NB / 4; ++t) {
        s_b[e16 * NB + 4 * t + g] = bq[t];
        s_bd[e16 * NB + 4 * t + g] = bd[t];
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);           // lgkmcnt(0): own LDS writes done (one wave)
      __builtin_amdgcn_wave_barrier();
      if (lane < NH) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p0 = s_dp[e * HS + lane], p1 = s_da[e * HS + lane];
#pragma unroll
          for (int n = 0; n < NB; ++n) w1[n] = fmaf(s_b[e * NB + n], p0, fmaf(s_bd[e * NB + n], p1, w1[n]));
        }
      }
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

// d_W2 pass, chunk-major as k_radial_bwd_w2 (one launch per term):
//   KIND 0: the weights' cotangent dw = gw(gg_x, Y, g) + gw(x, gg_Y, g),
//           contracted with the hidden values h;
//   KIND 1: the tangent's cotangent dv = gw(x, Y, g), contracted with the
//           hidden tangent gg_r SiLU'(pre) a.
// Each launch writes its own per-workgroup partials; like k_radial_bwd_w2 a
// launch covers the paths P0 .. P0 + NPG - 1 (wide signatures run one launch
// per path group, each writing its own columns).
template <class S, int U, int NB, int NH, int KIND, int P0 = 0, int NPG = S::NP>
__global__ void __launch_bounds__(64 * (NH / 16)) __attribute__((amdgpu_waves_per_eu(2)))
    k_radial_dbl_w2(int n_nodes, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col,
                    const float* __restrict__ x, const float* __restrict__ ggx, const float* __restrict__ Y,
                    const float* __restrict__ ggY, const float* __restrict__ r_len,
                    const float* __restrict__ ggr, RadialParams rp, const float* __restrict__ gout,
                    float* __restrict__ part, const int32_t* __restrict__ order) {
  static_assert(U % 16 == 0 && NH % 16 == 0 && NB % 4 == 0, "radial tiling");
  static_assert(P0 >= 0 && NPG > 0 && P0 + NPG <= S::NP, "path group");
  constexpr int NW = NH / 16;
  constexpr int LD = S::NP * U;
  constexpr int RS = 20, PS = 16 * RS;
  constexpr int TILE = NPG * PS;
  __shared__ __attribute__((aligned(16))) float s_gw[NW * TILE];
  __shared__ float s_r[NW * 16];                    // edge lengths of the tiles (-1: no edge)
  __shared__ float s_g[NW * 16];                    // their length cotangents (tangent term)
  const int c = blockIdx.y;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int e16 = lane & 15, g = lane >> 4;
  const int u = 16 * c + e16;
  f32x4 acc[NPG];
#pragma unroll
  for (int p = 0; p < NPG; ++p) acc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
  float w1b[NB / 4];
#pragma unroll
  for (int s = 0; s < NB / 4; ++s) w1b[s] = rp.W1[(4 * s + g) * NH + 16 * wv + e16];
  const float cb = sqrtf(2.0f / rp.r_cut);
  const float kk = 3.14159265358979323846f / rp.r_cut;
  const int stride = gridDim.x * NW;
  int pos = blockIdx.x * NW + wv, i = 0, t0 = 0, end = 0;   // position of the launch order, its node
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
        s_r[wv * 16 + e16] = q < end ? r_len[q] : -1.f;
        if constexpr (KIND == 1) s_g[wv * 16 + e16] = (q < end && ggr) ? ggr[q] : 0.f;
      }
      float gr[S::OC];
      load_o_channel<S, U>(gout, i, u, gr);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int q = t0 + 4 * g + r;
        const int qc = q < end ? q : end - 1;       // its hidden values are zero
        const int j = col[qc];
        float xr[S::XC], yr[S::YC], gxr[S::XC], gyr[S::YC];
        load_x_channel<S, U>(x, j, u, xr);
#pragma unroll
        for (int b = 0; b < S::YC; ++b) yr[b] = Y[(size_t)qc * S::YC + b];
        if constexpr (KIND == 0) {
          if (ggx) {
            load_x_channel<S, U>(ggx, j, u, gxr);
          } else {
#pragma unroll
            for (int a = 0; a < S::XC; ++a) gxr[a] = 0.f;
          }
#pragma unroll
          for (int b = 0; b < S::YC; ++b) gyr[b] = ggY ? ggY[(size_t)qc * S::YC + b] : 0.f;
        }
        static_for<NPG>([&](auto G) {
          constexpr PathInfo pi = S::paths.p[P0 + G];
          constexpr int D2 = 2 * pi.l2 + 1;
          float zx[D2];
          zform_scaled<pi.l1, pi.l2, pi.l3, pi.xo, pi.ko>(xr, gr, zx);
          float s = 0.f;
          if constexpr (KIND == 0) {
            float zg[D2];
            zform_scaled<pi.l1, pi.l2, pi.l3, pi.xo, pi.ko>(gxr, gr, zg);
            static_for<D2>([&](auto B2) {
              s = fmaf(yr[pi.yo + B2], zg[B2], s);
              s = fmaf(gyr[pi.yo + B2], zx[B2], s);
            });
          } else {
            static_for<D2>([&](auto B2) { s = fmaf(yr[pi.yo + B2], zx[B2], s); });
          }
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
      if (g == 0) {
        s_r[wv * 16 + e16] = -1.f;
        s_g[wv * 16 + e16] = 0.f;
      }
      for (int t = lane; t < TILE; t += 64) gw_own[t] = 0.f;
    }
    __syncthreads();
#pragma unroll 1
    for (int tw = 0; tw < NW; ++tw) {
      const float r = s_r[tw * 16 + e16];
      const bool v = r >= 0.f;
      const float rr = v ? r : 1.0f;
      const float inv = 1.0f / rr;
      f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f}, za = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NB / 4; ++s) {
        const float kn = (float)(4 * s + g + 1) * kk;
        const float sn = sinf(kn * rr);
        const float bn = v ? cb * sn * inv : 0.f;
        z = mfma_16x16x4(bn, w1b[s], z);
        if constexpr (KIND == 1) {
          const float bdn = v ? cb * (kn * cosf(kn * rr) * inv - sn * inv * inv) : 0.f;
          za = mfma_16x16x4(bdn, w1b[s], za);
        }
      }
      // z[t] = pre[edge 4g + t][hid 16w + e16], za[t] its derivative in r
      float hA[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float sg = sigmoid_fast(z[t]);
        if constexpr (KIND == 0) hA[t] = z[t] * sg;
        else hA[t] = s_g[tw * 16 + 4 * g + t] * silu_d1(z[t], sg) * za[t];
      }
      const float* gtl = s_gw + tw * TILE + 4 * g * RS + e16;
#pragma unroll
      for (int p = 0; p < NPG; ++p)
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[p] = mfma_16x16x4(hA[k], gtl[p * PS + k * RS], acc[p]);
    }
    __syncthreads();
  }
  float* pb = part + (size_t)blockIdx.x * NH * LD;
#pragma unroll
  for (int p = 0; p < NPG; ++p)
#pragma unroll
    for (int t = 0; t < 4; ++t) pb[(size_t)(16 * wv + 4 * g + t) * LD + (P0 + p) * U + u] = acc[p][t];
}

}  // namespace tpc
