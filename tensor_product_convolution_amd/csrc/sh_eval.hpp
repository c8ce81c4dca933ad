// Real spherical harmonics of an edge direction and their pullback to the
// edge vector, for one edge in registers (the second operand of the product:
// "The GPU Workload That Rewrites Molecular Physics", section "What Makes MLFF
// Workloads Structurally Different"; the gradient with respect to the edge
// vectors gives the forces a force field predicts, same page, opening
// sections).
//
// Component normalisation (sum_m Y_lm^2 = 2l + 1), real components m = -l..l
// built from Condon-Shortley complex harmonics, so for a unit direction
// (x, y, z): Y_0 = 1 and Y_1 = sqrt3 (y, z, x).  The polynomials are the
// standard real harmonics of degree <= 3 scaled by sqrt(4 pi).
//
// Contraction of a * b + c into fused multiply-adds is switched off in the
// direction and the harmonics: every operation rounds as written, so the
// harmonics are the same float32 values wherever they are inlined, whatever
// the surrounding code lets the compiler share.  The pullback (a gradient,
// compared to a tolerance, not bit for bit) may contract.
#pragma once
#include <hip/hip_runtime.h>

namespace tpc {

// (x, y, z) <- r / |r|, inv <- 1 / |r|; returns |r|.  1/|r| is the hardware
// reciprocal square root (about 1 ulp), |r| = |r|^2 / |r|; a vector whose
// squared length is below the smallest normal float counts as zero (all three
// results 0).
__device__ __forceinline__ float unit_dir(float& x, float& y, float& z, float& inv) {
#pragma clang fp contract(off)
  const float n2 = x * x + y * y + z * z;
  const bool nz = n2 >= 1.17549435e-38f;
  inv = nz ? __builtin_amdgcn_rsqf(n2) : 0.f;
  x *= inv;
  y *= inv;
  z *= inv;
  return n2 * inv;
}

// harmonics of the unit direction (x, y, z), (LMAX+1)^2 values
template <int LMAX, int N>
__device__ __forceinline__ void sh_eval(float x, float y, float z, float (&v)[N]) {
#pragma clang fp contract(off)
  static_assert(N >= (LMAX + 1) * (LMAX + 1), "room for every component");
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
}

// Pullback to the edge vector.  On the unit sphere each Y_lm is a homogeneous
// polynomial P_lm of degree l (the forms above with 1 replaced by
// x^2 + y^2 + z^2), and for Y(r) = P(r / |r|)
//   dY/dr = (grad P(u) - l P(u) u) / |r|,   u = r / |r|
// (Euler's identity u . grad P = l P makes it orthogonal to u).  Given the
// unit direction, 1/|r| and g = dL/dY, returns dL/dr = sum_b g_b dY_b/dr,
// plus gl u for a gradient gl with respect to the length |r|.
template <int LMAX, int N>
__device__ __forceinline__ void sh_pullback(float x, float y, float z, float inv, const float (&g)[N],
                                                     float gl, float (&gr)[3]) {
  static_assert(N >= (LMAX + 1) * (LMAX + 1), "room for every component");
  float gx = 0.f, gy = 0.f, gz = 0.f, lp = 0.f;   // sum g grad P, sum g l P
  if constexpr (LMAX >= 1) {
    const float s3 = 1.7320508075688772f;
    gx += s3 * g[3];
    gy += s3 * g[1];
    gz += s3 * g[2];
    lp += s3 * (g[1] * y + g[2] * z + g[3] * x);
  }
  if constexpr (LMAX >= 2) {
    const float s15 = 3.8729833462074170f, s5h = 1.1180339887498949f;
    const float P4 = s15 * x * y, P5 = s15 * y * z, P6 = s5h * (2.f * z * z - x * x - y * y);
    const float P7 = s15 * x * z, P8 = 0.5f * s15 * (x * x - y * y);
    gx += g[4] * s15 * y + g[6] * (-2.f * s5h * x) + g[7] * s15 * z + g[8] * s15 * x;
    gy += g[4] * s15 * x + g[5] * s15 * z + g[6] * (-2.f * s5h * y) + g[8] * (-s15 * y);
    gz += g[5] * s15 * y + g[6] * (4.f * s5h * z) + g[7] * s15 * x;
    lp += 2.f * (g[4] * P4 + g[5] * P5 + g[6] * P6 + g[7] * P7 + g[8] * P8);
  }
  if constexpr (LMAX >= 3) {
    const float c70 = 2.0916500663351889f, c105 = 10.246950765959598f;
    const float c42 = 1.6201851746019651f, c7 = 1.3228756555322954f;
    const float xx = x * x, yy = y * y, zz = z * z;
    const float P9 = c70 * y * (3.f * xx - yy), P10 = c105 * x * y * z;
    const float P11 = c42 * y * (4.f * zz - xx - yy), P12 = c7 * z * (2.f * zz - 3.f * xx - 3.f * yy);
    const float P13 = c42 * x * (4.f * zz - xx - yy), P14 = 0.5f * c105 * z * (xx - yy);
    const float P15 = c70 * x * (xx - 3.f * yy);
    gx += g[9] * c70 * 6.f * x * y + g[10] * c105 * y * z + g[11] * c42 * (-2.f * x * y) +
          g[12] * c7 * (-6.f * x * z) + g[13] * c42 * (4.f * zz - 3.f * xx - yy) +
          g[14] * c105 * x * z + g[15] * c70 * (3.f * xx - 3.f * yy);
    gy += g[9] * c70 * (3.f * xx - 3.f * yy) + g[10] * c105 * x * z +
          g[11] * c42 * (4.f * zz - xx - 3.f * yy) + g[12] * c7 * (-6.f * y * z) +
          g[13] * c42 * (-2.f * x * y) + g[14] * (-c105 * y * z) + g[15] * c70 * (-6.f * x * y);
    gz += g[10] * c105 * x * y + g[11] * c42 * 8.f * y * z + g[12] * c7 * (6.f * zz - 3.f * xx - 3.f * yy) +
          g[13] * c42 * 8.f * x * z + g[14] * 0.5f * c105 * (xx - yy);
    lp += 3.f * (g[9] * P9 + g[10] * P10 + g[11] * P11 + g[12] * P12 + g[13] * P13 + g[14] * P14 +
                 g[15] * P15);
  }
  gr[0] = (gx - lp * x) * inv + gl * x;
  gr[1] = (gy - lp * y) * inv + gl * y;
  gr[2] = (gz - lp * z) * inv + gl * z;
}

}  // namespace tpc
