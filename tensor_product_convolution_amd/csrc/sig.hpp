// Compile-time description of one tensor-product signature: the degrees of
// the input irreps (in string order), lmax of the harmonics and lmax of the
// output.  Path order and output-irrep order follow the plan builder:
//   paths: input irrep i (string order), then l2 = 0..LSH, then
//          l3 = |l1-l2| .. min(l1+l2, LOUT); output irrep (l3, (-1)^(l1+l2))
//          for inputs of natural parity;
//   outputs: distinct (l3, parity), l3 ascending, even before odd; every path
//          landing on one output irrep is summed into it.
// "Per channel" offsets below count components of one channel u; a node row
// of U channels stores each irrep block as [U][2l+1].
#pragma once
#include <utility>

#include "cg_table.hpp"

namespace tpc {

struct PathInfo {
  int in, l1, l2, l3, k;   // input irrep, degrees, output irrep index
  int xo, yo, ko;          // per-channel offsets of x block, Y block, out block
};

template <int MAXP>
struct PathArr {
  PathInfo p[MAXP];
};

struct OutInfo {
  int l, parity, ko;
};

template <int LSH, int LOUT, int... Ls>
struct Sig {
  static constexpr int NIN = sizeof...(Ls);
  static constexpr int lmax_sh = LSH;
  static constexpr int lmax_out = LOUT;
  struct LArr {
    int v[NIN];
  };
  static constexpr LArr ls{{Ls...}};
  static constexpr int XC = ((2 * Ls + 1) + ...);
  static constexpr int YC = (LSH + 1) * (LSH + 1);

  static constexpr int count_paths() {
    int n = 0;
    for (int i = 0; i < NIN; ++i)
      for (int l2 = 0; l2 <= LSH; ++l2) {
        int l1 = ls.v[i];
        int lo = l1 > l2 ? l1 - l2 : l2 - l1;
        int hi = l1 + l2 < LOUT ? l1 + l2 : LOUT;
        for (int l3 = lo; l3 <= hi; ++l3) ++n;
      }
    return n;
  }
  static constexpr int NP = count_paths();

  // output irreps present: slot (l, parity) -> used?
  static constexpr bool out_used(int l, int par) {
    for (int i = 0; i < NIN; ++i)
      for (int l2 = 0; l2 <= LSH; ++l2) {
        int l1 = ls.v[i];
        int lo = l1 > l2 ? l1 - l2 : l2 - l1;
        int hi = l1 + l2 < LOUT ? l1 + l2 : LOUT;
        int p = ((l1 + l2) & 1) ? -1 : 1;
        if (l >= lo && l <= hi && p == par) return true;
      }
    return false;
  }
  static constexpr int count_outs() {
    int n = 0;
    for (int l = 0; l <= LOUT; ++l) {
      if (out_used(l, 1)) ++n;
      if (out_used(l, -1)) ++n;
    }
    return n;
  }
  static constexpr int NO = count_outs();
  struct OArr {
    OutInfo o[NO];
  };
  static constexpr OArr make_outs() {
    OArr a{};
    int n = 0, ko = 0;
    for (int l = 0; l <= LOUT; ++l)
      for (int par = 1; par >= -1; par -= 2)
        if (out_used(l, par)) {
          a.o[n].l = l;
          a.o[n].parity = par;
          a.o[n].ko = ko;
          ko += 2 * l + 1;
          ++n;
        }
    return a;
  }
  static constexpr OArr outs = make_outs();
  static constexpr int OC = outs.o[NO - 1].ko + 2 * outs.o[NO - 1].l + 1;

  static constexpr int out_index(int l, int par) {
    for (int k = 0; k < NO; ++k)
      if (outs.o[k].l == l && outs.o[k].parity == par) return k;
    return -1;
  }

  static constexpr PathArr<NP> make_paths() {
    PathArr<NP> a{};
    int n = 0, xo = 0;
    for (int i = 0; i < NIN; ++i) {
      int l1 = ls.v[i];
      for (int l2 = 0; l2 <= LSH; ++l2) {
        int lo = l1 > l2 ? l1 - l2 : l2 - l1;
        int hi = l1 + l2 < LOUT ? l1 + l2 : LOUT;
        for (int l3 = lo; l3 <= hi; ++l3) {
          int k = out_index(l3, ((l1 + l2) & 1) ? -1 : 1);
          a.p[n] = PathInfo{i, l1, l2, l3, k, xo, l2 * l2, outs.o[k].ko};
          ++n;
        }
      }
      xo += 2 * l1 + 1;
    }
    return a;
  }
  static constexpr PathArr<NP> paths = make_paths();

  static constexpr int nnz_total() {
    int n = 0;
    for (int p = 0; p < NP; ++p) n += real_cg_nnz(paths.p[p].l1, paths.p[p].l2, paths.p[p].l3);
    return n;
  }

  // per-channel offset of input irrep i
  static constexpr int xoff(int i) {
    int o = 0;
    for (int t = 0; t < i; ++t) o += 2 * ls.v[t] + 1;
    return o;
  }
};

// ---------------------------------------------------------------------------
// compile-time loops with constant indices
template <class F, int... I>
__host__ __device__ __forceinline__ constexpr void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__host__ __device__ __forceinline__ constexpr void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

}  // namespace tpc
