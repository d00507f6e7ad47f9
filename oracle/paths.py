"""Admissible coupling paths and array layouts.

FlashCart paper, §2 "Irreducible Cartesian tensors": a path (l1, l2) -> l3 is
admissible when |l1 - l2| <= l3 <= l1 + l2 and l1 + l2 + l3 is even, i.e. the
product has natural parity (-1)^l3.  Node features carry the natural-parity
irreps l1 = 0..l1max (0e, 1o, 2e, 3o), edge harmonics l2 = 0..sh_lmax, and the
output keeps l3 <= out_lmax.  Paths are listed in lexicographic (l1, l2, l3)
order, which fixes the radial-weight column order p*C + u.

Layout (FlashCart §4 "Data layout": one contiguous block per rank, lower
ranks first, channels contiguous):
  h   [N][d_in][C]   l1 blocks ascending, m1 = -l1..l1 inside a block
  out [N][d_out][C]  l3 blocks ascending; inside the l3 block the order is
                     (m3, q, channel) where q ranks the paths with that l3

Path-summed output (FlashCart §3 "Generating Cartesian tensor products": the
kernels may sum the paths that share an output rank): every path with a
given l3 adds into one row block, so d_out = sum over the l3 values that
occur of (2 l3 + 1), with (m3, channel) order inside a block.
"""
from __future__ import annotations

from dataclasses import dataclass, field


def admissible(l1, l2, l3):
    return abs(l1 - l2) <= l3 <= l1 + l2 and (l1 + l2 + l3) % 2 == 0


def path_list(l1max, sh_lmax, out_lmax):
    return [(l1, l2, l3)
            for l1 in range(l1max + 1)
            for l2 in range(sh_lmax + 1)
            for l3 in range(out_lmax + 1)
            if admissible(l1, l2, l3)]


@dataclass
class Layout:
    l1max: int
    sh_lmax: int
    out_lmax: int
    C: int
    sum_paths: bool = False
    paths: list = field(init=False)

    def __post_init__(self):
        self.paths = path_list(self.l1max, self.sh_lmax, self.out_lmax)

    @property
    def n_paths(self):
        return len(self.paths)

    @property
    def d_in(self):
        return (self.l1max + 1) ** 2

    @property
    def d_sh(self):
        return (self.sh_lmax + 1) ** 2

    def _out_l3(self):
        return sorted({l3 for (_, _, l3) in self.paths})

    @property
    def d_out(self):
        if self.sum_paths:
            return sum(2 * l3 + 1 for l3 in self._out_l3())
        return sum(2 * l3 + 1 for (_, _, l3) in self.paths)

    def in_slice(self, l1):
        return slice(l1 * l1, (l1 + 1) * (l1 + 1))

    def sh_slice(self, l2):
        return slice(l2 * l2, (l2 + 1) * (l2 + 1))

    def out_rows(self, p):
        """Output row index of (path p, m3) for m3 = 0..2 l3."""
        l3 = self.paths[p][2]
        if self.sum_paths:
            base = sum(2 * l + 1 for l in self._out_l3() if l < l3)
            return [base + m3 for m3 in range(2 * l3 + 1)]
        base = sum((2 * l + 1) * sum(1 for q in self.paths if q[2] == l)
                   for l in range(l3))
        same = [k for k, q in enumerate(self.paths) if q[2] == l3]
        q = same.index(p)
        return [base + m3 * len(same) + q for m3 in range(2 * l3 + 1)]
