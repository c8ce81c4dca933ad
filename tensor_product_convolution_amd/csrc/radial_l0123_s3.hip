// Radial-weight kernel specialisations for the 0e+1o+2e+3o / lmax 3 signature
// (34 paths).  The chunk's W2 slice takes 140 KB of LDS, so one workgroup fits
// a CU: the forward and the sender pass run four waves (one per SIMD, 256
// registers and up to 220 accumulation registers each), the receiver pass
// eight waves that share the slice (two per SIMD at 256 registers, with a few
// spilled: 1.03 against 1.37 ms with four waves on 4,096 atoms at 64
// channels, the latency of each path's LDS -> MFMA -> VALU -> MFMA chain
// hidden by the second wave).  grad_W2 and the two d_W2 terms of the
// second-order pass run in three launches of at most 12 paths each.  The
// second-order node and receiver passes hold more state than a wave's 512
// registers at 34 paths and spill (one wave per SIMD).
#include "radial_launch.hpp"

namespace tpc {

using RadialL0123 = RadialSig<Sig<3, 3, 0, 1, 2, 3>, 12, 8, true>;

const RadialSet* radial_l0123_s3(int mul, int nb, int nh) {
  if (nb != kNB || nh != kNH) return nullptr;
  switch (mul) {
    case 16: return radial_set<RadialL0123, 16>();
    case 32: return radial_set<RadialL0123, 32>();
    case 64: return radial_set<RadialL0123, 64>();
    default: return nullptr;
  }
}

}  // namespace tpc
