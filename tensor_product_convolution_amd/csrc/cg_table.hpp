// Clebsch-Gordan tables for the real-basis tensor product, computable both at
// compile time (kernel specialisations carry the nonzeros as immediates) and
// at run time (the plan builder exposes them for inspection).
//
// The pages name the sparse CG product and its path aggregation ("FlashTP:
// Fused, Sparsity-Aware Tensor Product for MLIPs", Abstract) but print no
// coefficient or convention.  Conventions implemented here:
//   * complex CG from Racah's closed form, Condon-Shortley phase;
//   * real components m = -l..l from the usual real/complex combination
//     (l = 1 components come out as (y, z, x));
//   * the real tensor of a path is purely real (l1+l2+l3 even) or purely
//     imaginary (odd) after the change of basis; the nonzero part is taken;
//   * |C| <= 1e-12 is a zero; the sign makes the lexicographically first
//     nonzero (a, b, c) positive; sum_ab C[a,b,c] C[a,b,c'] = delta_cc'.
#pragma once
#include <cstdint>

namespace tpc {

constexpr int kMaxL = 6;          // largest degree the table builder accepts
constexpr double kZeroTol = 1e-12;

constexpr double cx_sqrt(double a) {
  if (a <= 0.0) return 0.0;
  double x = a >= 1.0 ? a : 1.0;
  for (int i = 0; i < 200; ++i) {
    double nx = 0.5 * (x + a / x);
    if (nx == x) break;
    x = nx;
  }
  // settle on the better of the two neighbours the iteration can cycle on
  double y = 0.5 * (x + a / x);
  double ex = x * x - a, ey = y * y - a;
  return (ex < 0 ? -ex : ex) <= (ey < 0 ? -ey : ey) ? x : y;
}

constexpr double cx_fact(int n) {
  double r = 1.0;
  for (int i = 2; i <= n; ++i) r *= static_cast<double>(i);
  return r;
}

constexpr int cx_abs(int v) { return v < 0 ? -v : v; }

// <j1 m1 j2 m2 | J M>, integer momenta.
constexpr double cg_complex(int j1, int m1, int j2, int m2, int J, int M) {
  if (M != m1 + m2) return 0.0;
  if (J < cx_abs(j1 - j2) || J > j1 + j2) return 0.0;
  if (cx_abs(m1) > j1 || cx_abs(m2) > j2 || cx_abs(M) > J) return 0.0;
  double pre = (2.0 * J + 1.0) * cx_fact(J + j1 - j2) * cx_fact(J - j1 + j2) *
               cx_fact(j1 + j2 - J) / cx_fact(j1 + j2 + J + 1);
  pre *= cx_fact(J + M) * cx_fact(J - M) * cx_fact(j1 - m1) * cx_fact(j1 + m1) *
         cx_fact(j2 - m2) * cx_fact(j2 + m2);
  int kmin = 0;
  if (j2 - J - m1 > kmin) kmin = j2 - J - m1;
  if (j1 - J + m2 > kmin) kmin = j1 - J + m2;
  int kmax = j1 + j2 - J;
  if (j1 - m1 < kmax) kmax = j1 - m1;
  if (j2 + m2 < kmax) kmax = j2 + m2;
  double s = 0.0;
  for (int k = kmin; k <= kmax; ++k) {
    double den = cx_fact(k) * cx_fact(j1 + j2 - J - k) * cx_fact(j1 - m1 - k) *
                 cx_fact(j2 + m2 - k) * cx_fact(J - j2 + m1 + k) * cx_fact(J - j1 - m2 + k);
    s += ((k & 1) ? -1.0 : 1.0) / den;
  }
  return cx_sqrt(pre) * s;
}

struct Cx {
  double re = 0.0, im = 0.0;
};
constexpr Cx cx_mul(Cx a, Cx b) { return {a.re * b.re - a.im * b.im, a.re * b.im + a.im * b.re}; }
constexpr Cx cx_conj(Cx a) { return {a.re, -a.im}; }

// Entry of the real-basis matrix: row a (real component m = a - l), column
// mc (complex m = mc - l).
constexpr Cx real_basis(int l, int a, int mc) {
  const double r2 = 0.70710678118654752440;  // 1/sqrt(2)
  int m = a - l, mm = mc - l;
  if (m == 0) return mm == 0 ? Cx{1.0, 0.0} : Cx{};
  if (m > 0) {
    if (mm == m) return Cx{(m & 1) ? -r2 : r2, 0.0};
    if (mm == -m) return Cx{r2, 0.0};
    return Cx{};
  }
  // m < 0
  if (mm == m) return Cx{0.0, r2};
  if (mm == -m) return Cx{0.0, ((-m) & 1) ? r2 : -r2};
  return Cx{};
}

// Real CG entry before the sign rule; `parity_imag` picks the imaginary part.
constexpr double real_cg_raw(int l1, int l2, int l3, int a, int b, int c) {
  Cx z{};
  // each real component mixes only +-m, so only two complex columns per row
  int ma = a - l1, mb = b - l2, mcc = c - l3;
  int cols1[2] = {ma + l1, -ma + l1};
  int cols2[2] = {mb + l2, -mb + l2};
  int cols3[2] = {mcc + l3, -mcc + l3};
  int n1 = ma == 0 ? 1 : 2, n2 = mb == 0 ? 1 : 2, n3 = mcc == 0 ? 1 : 2;
  for (int i = 0; i < n1; ++i)
    for (int j = 0; j < n2; ++j)
      for (int k = 0; k < n3; ++k) {
        int m1 = cols1[i] - l1, m2 = cols2[j] - l2, m3 = cols3[k] - l3;
        if (m1 + m2 != m3) continue;
        double cg = cg_complex(l1, m1, l2, m2, l3, m3);
        if (cg == 0.0) continue;
        Cx t = cx_mul(cx_mul(cx_conj(real_basis(l1, a, cols1[i])),
                             cx_conj(real_basis(l2, b, cols2[j]))),
                      real_basis(l3, c, cols3[k]));
        z.re += t.re * cg;
        z.im += t.im * cg;
      }
  return ((l1 + l2 + l3) & 1) ? z.im : z.re;
}

constexpr bool triangle(int l1, int l2, int l3) {
  return l3 >= cx_abs(l1 - l2) && l3 <= l1 + l2;
}

// Sign (+1 / -1) of the path's real tensor under the first-nonzero rule.
constexpr double real_cg_sign(int l1, int l2, int l3) {
  for (int a = 0; a <= 2 * l1; ++a)
    for (int b = 0; b <= 2 * l2; ++b)
      for (int c = 0; c <= 2 * l3; ++c) {
        double v = real_cg_raw(l1, l2, l3, a, b, c);
        if (v > kZeroTol) return 1.0;
        if (v < -kZeroTol) return -1.0;
      }
  return 1.0;
}

constexpr double real_cg(int l1, int l2, int l3, int a, int b, int c, double sign) {
  double v = real_cg_raw(l1, l2, l3, a, b, c);
  if (v <= kZeroTol && v >= -kZeroTol) return 0.0;
  return sign * v;
}

constexpr int real_cg_nnz(int l1, int l2, int l3) {
  if (!triangle(l1, l2, l3)) return 0;
  int n = 0;
  for (int a = 0; a <= 2 * l1; ++a)
    for (int b = 0; b <= 2 * l2; ++b)
      for (int c = 0; c <= 2 * l3; ++c) {
        double v = real_cg_raw(l1, l2, l3, a, b, c);
        if (v > kZeroTol || v < -kZeroTol) ++n;
      }
  return n;
}

struct Nz {
  int8_t a, b, c;
  float v;
};

// Compile-time nonzero list of one path, lexicographic (a, b, c) order.
template <int L1, int L2, int L3>
struct CgPath {
  static constexpr int nnz = real_cg_nnz(L1, L2, L3);
  struct Table {
    Nz e[nnz > 0 ? nnz : 1];
  };
  static constexpr Table make() {
    Table t{};
    double s = real_cg_sign(L1, L2, L3);
    int n = 0;
    for (int a = 0; a <= 2 * L1; ++a)
      for (int b = 0; b <= 2 * L2; ++b)
        for (int c = 0; c <= 2 * L3; ++c) {
          double v = real_cg(L1, L2, L3, a, b, c, s);
          if (v != 0.0) {
            t.e[n].a = static_cast<int8_t>(a);
            t.e[n].b = static_cast<int8_t>(b);
            t.e[n].c = static_cast<int8_t>(c);
            t.e[n].v = static_cast<float>(v);
            ++n;
          }
        }
    return t;
  }
  static constexpr Table table = make();
  // does some nonzero couple Y component b to output component c?
  static constexpr bool has_bc(int b, int c) {
    for (int n = 0; n < nnz; ++n)
      if (table.e[n].b == b && table.e[n].c == c) return true;
    return false;
  }
};

}  // namespace tpc
