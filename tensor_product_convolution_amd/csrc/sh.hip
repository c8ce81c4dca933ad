// Real spherical harmonics of edge directions and their gradient with respect
// to the edge vectors, one thread per edge (the polynomials and their
// pullback are in sh_eval.hpp, shared with the kernels that evaluate the
// harmonics on chip).
#include "internal.hpp"
#include "sh_eval.hpp"

namespace tpc {
namespace {

template <int LMAX>
__global__ void __launch_bounds__(256)
    k_sph_harm(const float* __restrict__ r, int n, float* __restrict__ Y) {
  constexpr int YC = (LMAX + 1) * (LMAX + 1);
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  float x = r[3 * (size_t)e], y = r[3 * (size_t)e + 1], z = r[3 * (size_t)e + 2], inv;
  unit_dir(x, y, z, inv);
  float v[YC];
  sh_eval<LMAX>(x, y, z, v);
#pragma unroll
  for (int t = 0; t < YC; ++t) Y[(size_t)e * YC + t] = v[t];
}

// Gradient with respect to the edge vector (sh_pullback): grad_r = sum_b
// grad_Y[b] dY_b/dr, plus grad_rlen * u when the edge length also feeds the
// layer (radial weights).
template <int LMAX>
__global__ void __launch_bounds__(256)
    k_sph_harm_bwd(const float* __restrict__ r, int n, const float* __restrict__ gY,
                   const float* __restrict__ grl, float* __restrict__ gr) {
  constexpr int YC = (LMAX + 1) * (LMAX + 1);
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  float x = r[3 * (size_t)e], y = r[3 * (size_t)e + 1], z = r[3 * (size_t)e + 2], inv;
  unit_dir(x, y, z, inv);
  float g[YC];
#pragma unroll
  for (int t = 0; t < YC; ++t) g[t] = gY[(size_t)e * YC + t];
  float o[3];
  sh_pullback<LMAX>(x, y, z, inv, g, grl ? grl[e] : 0.f, o);
  gr[3 * (size_t)e + 0] = o[0];
  gr[3 * (size_t)e + 1] = o[1];
  gr[3 * (size_t)e + 2] = o[2];
}

}  // namespace

tp_status sph_harm_bwd(int lmax, const float* r, int n, const float* gY, const float* grl, float* gr,
                       hipStream_t st) {
  if (n == 0) return TP_OK;
  const dim3 grid((n + 255) / 256), block(256);
  switch (lmax) {
    case 0: hipLaunchKernelGGL(k_sph_harm_bwd<0>, grid, block, 0, st, r, n, gY, grl, gr); break;
    case 1: hipLaunchKernelGGL(k_sph_harm_bwd<1>, grid, block, 0, st, r, n, gY, grl, gr); break;
    case 2: hipLaunchKernelGGL(k_sph_harm_bwd<2>, grid, block, 0, st, r, n, gY, grl, gr); break;
    case 3: hipLaunchKernelGGL(k_sph_harm_bwd<3>, grid, block, 0, st, r, n, gY, grl, gr); break;
    default: return set_error(TP_ERR_UNSUPPORTED, "tp_conv_sph_harm_backward: lmax must be 0..3");
  }
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? TP_OK : hip_error(e, "sph_harm_bwd launch");
}

tp_status sph_harm(int lmax, const float* r, int n, float* Y, hipStream_t st) {
  if (n == 0) return TP_OK;
  const dim3 grid((n + 255) / 256), block(256);
  switch (lmax) {
    case 0: hipLaunchKernelGGL(k_sph_harm<0>, grid, block, 0, st, r, n, Y); break;
    case 1: hipLaunchKernelGGL(k_sph_harm<1>, grid, block, 0, st, r, n, Y); break;
    case 2: hipLaunchKernelGGL(k_sph_harm<2>, grid, block, 0, st, r, n, Y); break;
    case 3: hipLaunchKernelGGL(k_sph_harm<3>, grid, block, 0, st, r, n, Y); break;
    default: return set_error(TP_ERR_UNSUPPORTED, "tp_conv_sph_harm: lmax must be 0..3");
  }
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? TP_OK : hip_error(e, "sph_harm launch");
}

}  // namespace tpc
