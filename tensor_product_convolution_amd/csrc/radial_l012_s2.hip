// Radial-weight kernel specialisations for the 0e+1o+2e / lmax 2 signature.
#include "radial_kernels.hpp"

namespace tpc {

using SigR = Sig<2, 2, 0, 1, 2>;

template <int U>
static hipError_t launch_radial_fwd(const RadialArgs& a) {
  if (a.n_nodes == 0) return hipSuccess;
  RadialParams rp{a.r_cut, a.W1, a.W2};
  hipLaunchKernelGGL((k_radial_fwd<SigR, U, 8, 64>), dim3(a.n_nodes), dim3(64), 0, a.stream,
                     a.row_ptr, a.col, a.x, a.Y, a.r_len, rp, a.out);
  return hipGetLastError();
}

template <int U>
static const RadialSet* radial_set() {
  static const RadialSet s{&launch_radial_fwd<U>, nullptr};
  return &s;
}

const RadialSet* radial_l012_s2(int mul, int nb, int nh) {
  if (nb != 8 || nh != 64) return nullptr;
  switch (mul) {
    case 16: return radial_set<16>();
    case 128: return radial_set<128>();
    default: return nullptr;
  }
}

}  // namespace tpc
