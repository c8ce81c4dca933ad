// Kernel specialisations for one tensor-product signature; see sig.hpp for
// the meaning of the template arguments (lmax_sh, lmax_out, input degrees).
#include "conv_kernels.hpp"

namespace tpc {

using Sig_l0123_s3 = Sig<3, 3, 0, 1, 2, 3>;

const KernelSet* kernels_l0123_s3(int mul) {
  switch (mul) {
    case 8: return kernel_set<Sig_l0123_s3, 8>();
    case 16: return kernel_set<Sig_l0123_s3, 16>();
    case 32: return kernel_set<Sig_l0123_s3, 32>();
    case 64: return kernel_set<Sig_l0123_s3, 64>();
    case 128: return kernel_set<Sig_l0123_s3, 128>();
    default: return nullptr;
  }
}

}  // namespace tpc
