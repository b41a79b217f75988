"""Irreps strings and path enumeration (oracle side; test infrastructure).

Notation follows the configurations of the CGTP convolution ("32x0e+32x1o"):
a sum of terms ``[mul x] l parity``.  The pages only use this notation; the
admissibility rules below are the textbook ones for an O(3)-equivariant
coupling:

  * triangle rule |l1 - l2| <= l3 <= l1 + l2,
  * parity rule p1 * (-1)**l2 == p3 (spherical harmonics of order l have
    parity (-1)**l),
  * channelwise (uvu) coupling needs mul(s1) == mul(s3).

Paths are listed in lexicographic (s1, l2, s3) order; this order is the
column layout of the per-edge weights W: path p occupies columns
[sum_{q<p} mul_q, sum_{q<=p} mul_q).
"""

from __future__ import annotations

import re
from dataclasses import dataclass
from typing import List, Tuple

_TERM = re.compile(r"^\s*(?:(\d+)\s*x\s*)?(\d+)\s*([eo])\s*$")


@dataclass(frozen=True)
class Irrep:
    mul: int
    l: int
    p: int  # +1 even, -1 odd

    @property
    def dim(self) -> int:
        return self.mul * (2 * self.l + 1)


class Irreps(tuple):
    """A tuple of Irrep segments with offsets into a concatenated feature row."""

    @property
    def dim(self) -> int:
        return sum(s.dim for s in self)

    def offsets(self) -> List[int]:
        off, res = 0, []
        for s in self:
            res.append(off)
            off += s.dim
        return res

    def slice(self, s: int) -> slice:
        o = self.offsets()[s]
        return slice(o, o + self[s].dim)


def parse_irreps(text: str) -> Irreps:
    """Parse ``term('+'term)*`` with ``term = [mul 'x'] l ('e'|'o')``."""
    if not isinstance(text, str) or not text.strip():
        raise ValueError(f"empty irreps string: {text!r}")
    segs = []
    for term in text.split("+"):
        m = _TERM.match(term)
        if not m:
            raise ValueError(f"bad irreps term {term!r} in {text!r}")
        mul = int(m.group(1)) if m.group(1) is not None else 1
        if mul <= 0:
            raise ValueError(f"multiplicity must be positive in {text!r}")
        segs.append(Irrep(mul, int(m.group(2)), 1 if m.group(3) == "e" else -1))
    return Irreps(segs)


def enumerate_paths(irreps_in: Irreps, sh_lmax: int, irreps_out: Irreps) -> List[Tuple[int, int, int]]:
    """All admissible (s1, l2, s3), lexicographic.  Raises on a uvu mul mismatch."""
    paths = []
    for s1, a in enumerate(irreps_in):
        for l2 in range(sh_lmax + 1):
            for s3, c in enumerate(irreps_out):
                if not (abs(a.l - l2) <= c.l <= a.l + l2):
                    continue
                if a.p * (-1) ** l2 != c.p:
                    continue
                if a.mul != c.mul:
                    raise ValueError(
                        f"channelwise path {a.mul}x{a.l} x {l2} -> {c.mul}x{c.l} needs equal multiplicities")
                paths.append((s1, l2, s3))
    return paths
