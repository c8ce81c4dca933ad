// Radial-weight kernel specialisations for the 0e+1o+2e / lmax 2 signature.
#include "radial_launch.hpp"

namespace tpc {

// all 15 paths' grad_w tiles fit in one grad_W2 launch; receiver pass of four
// waves (two workgroups per CU); second order built
using RadialL012 = RadialSig<Sig<2, 2, 0, 1, 2>, 15, 4, true>;

const RadialSet* radial_l012_s2(int mul, int nb, int nh) {
  if (nb != kNB || nh != kNH) return nullptr;
  switch (mul) {
    case 16: return radial_set<RadialL012, 16>();
    case 32: return radial_set<RadialL012, 32>();
    case 64: return radial_set<RadialL012, 64>();
    case 128: return radial_set<RadialL012, 128>();
    default: return nullptr;
  }
}

}  // namespace tpc
