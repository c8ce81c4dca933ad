"""Irreps strings, the path set and the output irreps of a uvu tensor product.

Test infrastructure only (see ``oracle/__init__.py``).

The pages speak of path-aggregated execution over every (l1, l2 -> l3) path
("FlashTP: Fused, Sparsity-Aware Tensor Product for MLIPs", Abstract) and of
the NequIP convolution ("Accelerating Tensor Products in E(3)-Equivariant Graph
Neural Networks", Abstract) but fix no order or layout.  Readings:

* irreps are ``MxLp`` terms joined by ``+`` (p in {e, o}); channel-wise
  ("uvu") coupling needs one multiplicity U shared by all input irreps, and
  every input irrep has natural parity (-1)^L;
* paths: l1 over the input irreps in string order, then l2 = 0..lmax_sh, then
  l3 = |l1-l2| .. min(l1+l2, lmax_out); the triangle rule is the only filter;
* a path's output irrep is (l3, p1 * (-1)^l2);
* output irreps are the distinct (l3, parity) pairs, l3 ascending, ``e``
  before ``o``; all paths that land on one output irrep are summed into it;
* layouts: a node row is the concatenation of irrep blocks, each block
  ``[U][2l+1]`` (channel-major); Y rows are l-blocks with m = -l..l; the
  weights of an edge are ``[P][U]``.
"""
import re
from dataclasses import dataclass, field

import numpy as np

from .cg import cg_real

_TERM = re.compile(r"^\s*(\d+)x(\d+)([eo])\s*$")


def parse_irreps(s):
    """Parse ``"32x0e+32x1o"`` into a list of (mul, l, parity) with parity +-1."""
    out = []
    if not isinstance(s, str) or not s.strip():
        raise ValueError("empty irreps string")
    for term in s.split("+"):
        m = _TERM.match(term)
        if not m:
            raise ValueError(f"bad irreps term {term!r}")
        mul, l, p = int(m.group(1)), int(m.group(2)), m.group(3)
        if mul <= 0:
            raise ValueError(f"multiplicity must be positive in {term!r}")
        out.append((mul, l, 1 if p == "e" else -1))
    return out


def irreps_str(irreps):
    return "+".join(f"{m}x{l}{'e' if p == 1 else 'o'}" for m, l, p in irreps)


@dataclass
class OraclePlan:
    """Everything about a plan that the convolution needs, in float64."""
    irreps_in: list           # [(U, l, parity)]
    U: int
    lmax_sh: int
    lmax_out: int
    paths: list               # [(i_in, l1, l2, l3, k_out)]
    out_irreps: list          # [(l3, parity)]
    in_offsets: list          # start column of each input block in a node row
    out_offsets: list         # start column of each output block
    xdim: int
    outdim: int
    ysh: int
    cg: list = field(default_factory=list)   # per path: float64 C[a,b,c]

    @property
    def n_paths(self):
        return len(self.paths)

    def sh_slice(self, l):
        return slice(l * l, (l + 1) * (l + 1))

    def nnz(self):
        return int(sum(int(np.count_nonzero(C)) for C in self.cg))

    def out_irreps_str(self):
        return "+".join(f"{self.U}x{l}{'e' if p == 1 else 'o'}" for l, p in self.out_irreps)


def build_plan(irreps_in, lmax_sh, lmax_out):
    """Path list, output irreps, offsets and real CG tensors (readings above)."""
    irr = parse_irreps(irreps_in) if isinstance(irreps_in, str) else list(irreps_in)
    muls = {m for m, _, _ in irr}
    if len(muls) != 1:
        raise ValueError("uvu needs one multiplicity shared by all input irreps")
    for _, l, p in irr:
        if p != (-1) ** l:
            raise ValueError("input irreps must have natural parity (-1)^l")
    if lmax_sh < 0 or lmax_out < 0:
        raise ValueError("lmax must be >= 0")
    U = muls.pop()
    raw = []
    for i, (_, l1, p1) in enumerate(irr):
        for l2 in range(lmax_sh + 1):
            for l3 in range(abs(l1 - l2), min(l1 + l2, lmax_out) + 1):
                raw.append((i, l1, l2, l3, (l3, p1 * (-1) ** l2)))
    outs = sorted({r[4] for r in raw}, key=lambda lp: (lp[0], -lp[1]))
    kidx = {lp: k for k, lp in enumerate(outs)}
    paths = [(i, l1, l2, l3, kidx[lp]) for i, l1, l2, l3, lp in raw]
    in_off, o = [], 0
    for _, l, _ in irr:
        in_off.append(o)
        o += U * (2 * l + 1)
    xdim = o
    out_off, o = [], 0
    for l, _ in outs:
        out_off.append(o)
        o += U * (2 * l + 1)
    plan = OraclePlan(irreps_in=irr, U=U, lmax_sh=lmax_sh, lmax_out=lmax_out,
                      paths=paths, out_irreps=outs, in_offsets=in_off,
                      out_offsets=out_off, xdim=xdim, outdim=o,
                      ysh=(lmax_sh + 1) ** 2)
    plan.cg = [cg_real(l1, l2, l3) for _, l1, l2, l3, _ in paths]
    return plan
