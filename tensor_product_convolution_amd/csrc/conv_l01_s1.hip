// Kernel specialisations for one tensor-product signature; see sig.hpp for
// the meaning of the template arguments (lmax_sh, lmax_out, input degrees).
#include "conv_kernels.hpp"

namespace tpc {

using Sig_l01_s1 = Sig<1, 1, 0, 1>;

const KernelSet* kernels_l01_s1(int mul) {
  switch (mul) {
    case 8: return kernel_set<Sig_l01_s1, 8>();
    case 16: return kernel_set<Sig_l01_s1, 16>();
    case 32: return kernel_set<Sig_l01_s1, 32>();
    case 64: return kernel_set<Sig_l01_s1, 64>();
    case 128: return kernel_set<Sig_l01_s1, 128>();
    default: return nullptr;
  }
}

}  // namespace tpc
