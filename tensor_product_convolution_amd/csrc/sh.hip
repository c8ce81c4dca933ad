// Real spherical harmonics of edge directions (the second operand of the
// product: "The GPU Workload That Rewrites Molecular Physics", section "What
// Makes MLFF Workloads Structurally Different").
//
// Component normalisation (sum_m Y_lm^2 = 2l + 1), real components m = -l..l
// built from Condon-Shortley complex harmonics, so for a unit direction
// (x, y, z): Y_0 = 1 and Y_1 = sqrt3 (y, z, x).  The polynomials below are the
// standard real harmonics of degree <= 3 scaled by sqrt(4 pi).
#include "internal.hpp"

namespace tpc {
namespace {

template <int LMAX>
__global__ void __launch_bounds__(256)
    k_sph_harm(const float* __restrict__ r, int n, float* __restrict__ Y) {
  constexpr int YC = (LMAX + 1) * (LMAX + 1);
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  float x = r[3 * (size_t)e], y = r[3 * (size_t)e + 1], z = r[3 * (size_t)e + 2];
  const float n2 = x * x + y * y + z * z;
  const float inv = n2 > 0.f ? 1.0f / sqrtf(n2) : 0.f;
  x *= inv;
  y *= inv;
  z *= inv;
  float v[YC];
  v[0] = 1.0f;
  if constexpr (LMAX >= 1) {
    const float s3 = 1.7320508075688772f;
    v[1] = s3 * y;
    v[2] = s3 * z;
    v[3] = s3 * x;
  }
  if constexpr (LMAX >= 2) {
    const float s15 = 3.8729833462074170f, s5h = 1.1180339887498949f;
    v[4] = s15 * x * y;
    v[5] = s15 * y * z;
    v[6] = s5h * (3.f * z * z - 1.f);
    v[7] = s15 * x * z;
    v[8] = 0.5f * s15 * (x * x - y * y);
  }
  if constexpr (LMAX >= 3) {
    const float c70 = 2.0916500663351889f;   // sqrt(70)/4
    const float c105 = 10.246950765959598f;  // sqrt(105)
    const float c42 = 1.6201851746019651f;   // sqrt(42)/4
    const float c7 = 1.3228756555322954f;    // sqrt(7)/2
    const float z2 = z * z;
    v[9] = c70 * y * (3.f * x * x - y * y);
    v[10] = c105 * x * y * z;
    v[11] = c42 * y * (5.f * z2 - 1.f);
    v[12] = c7 * z * (5.f * z2 - 3.f);
    v[13] = c42 * x * (5.f * z2 - 1.f);
    v[14] = 0.5f * c105 * z * (x * x - y * y);
    v[15] = c70 * x * (x * x - 3.f * y * y);
  }
#pragma unroll
  for (int t = 0; t < YC; ++t) Y[(size_t)e * YC + t] = v[t];
}

}  // namespace

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
