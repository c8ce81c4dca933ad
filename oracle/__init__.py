"""Float64 CPU oracle for the E(3)-equivariant tensor-product graph convolution.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
GPU product path (``tensor_product_convolution_amd``) never imports, links or
runs it, and this package imports nothing from the product path: the two share
no code, tables, constants or pre/post-processing.

What it computes is the operator the pages describe in prose only:

* the NequIP equivariant convolution whose tensor product dominates the
  interaction layer ("Accelerating Tensor Products in E(3)-Equivariant Graph
  Neural Networks", NeurIPS 2026, Abstract);
* the full Clebsch-Gordan product, not a cheaper substitute, since different
  tensor products are different operations ("The Price of Freedom: Exploring
  Expressivity and Runtime Tradeoffs in Equivariant Tensor Products", ICML
  2025, Abstract);
* separately, the Gaunt product (the pointwise product of spherical signals,
  evaluated on a grid), which the same page sets apart as a cheaper and less
  expressive operation (``gaunt.py``);
* edge-conditioned, scatter-summed into receivers; edge-sized messages are a
  property of the schedule, not of the operator ("Sobek: Streaming Equivariant
  Tensor Product Convolutions", Abstract) -- so this oracle materialises
  per-edge messages freely, which the GPU path must not.

Every convention the pages leave open (real basis, CG phase and sign, path and
output order, normalisation, edge-vector direction, radial basis) is a stated
reading; each function's docstring names the reading it implements.

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
things other than itself (sympy's exact CG, scipy's spherical harmonics,
closed forms, Wigner-D equivariance, trilinearity, finite differences and
brute-force loops).  No function here is "parity unpinned".
"""
from .irreps import parse_irreps, build_plan, OraclePlan
from .cg import cg_complex, real_basis_matrix, cg_real
from .sh import sh_complex, sh_real, sh_real_jacobian, sh_real_vjp
from .wigner import wigner_D_real
from .csr import csr_build, launch_order
from .conv import (tp_conv_fwd, tp_conv_bwd, bessel_basis, bessel_basis_deriv, radial_mlp_fwd,
                   radial_mlp_bwd, uvw_mix_fwd, uvw_mix_bwd,
                   tp_conv_radial_fwd, tp_conv_radial_bwd, tp_conv_double_bwd,
                   bessel_basis_deriv2, silu_derivs, tp_conv_radial_double_bwd)
from .fc import fc_conv_fwd, fc_conv_bwd, fc_conv_double_bwd
from .gaunt import (sphere_quadrature, gaunt_coefficients, gaunt_plan, gaunt_conv_fwd,
                    gaunt_conv_bwd, gaunt_conv_double_bwd)

__all__ = [
    "parse_irreps", "build_plan", "OraclePlan", "cg_complex",
    "real_basis_matrix", "cg_real", "sh_complex", "sh_real", "sh_real_jacobian",
    "sh_real_vjp", "wigner_D_real", "csr_build", "launch_order", "tp_conv_fwd", "tp_conv_bwd",
    "bessel_basis", "bessel_basis_deriv",
    "radial_mlp_fwd", "radial_mlp_bwd", "uvw_mix_fwd", "uvw_mix_bwd",
    "tp_conv_radial_fwd", "tp_conv_radial_bwd", "tp_conv_double_bwd", "bessel_basis_deriv2",
    "silu_derivs", "tp_conv_radial_double_bwd", "fc_conv_fwd",
    "fc_conv_bwd", "fc_conv_double_bwd", "sphere_quadrature", "gaunt_coefficients", "gaunt_plan", "gaunt_conv_fwd",
    "gaunt_conv_bwd", "gaunt_conv_double_bwd",
]
