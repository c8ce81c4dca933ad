// Kernel specialisations for one tensor-product signature; see sig.hpp for
// the meaning of the template arguments (lmax_sh, lmax_out, input degrees).
#include "conv_kernels.hpp"

namespace tpc {

using Sig_l012_s2 = Sig<2, 2, 0, 1, 2>;

const KernelSet* kernels_l012_s2(int mul) {
  switch (mul) {
    case 8: return kernel_set<Sig_l012_s2, 8>();
    case 16: return kernel_set<Sig_l012_s2, 16>();
    case 32: return kernel_set<Sig_l012_s2, 32>();
    case 64: return kernel_set<Sig_l012_s2, 64>();
    case 128: return kernel_set<Sig_l012_s2, 128>();
    default: return nullptr;
  }
}

}  // namespace tpc
