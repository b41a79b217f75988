"""Seeded synthetic inputs for the CGTP convolution (shared by tests and bench).

This module is the only code that both the HIP path's callers and the oracle
consume.  It holds none of the convolution's arithmetic: it draws atom
positions, builds the neighbour list, evaluates the edges' real spherical
harmonics (an input of the convolution), and draws node features, per-edge
path weights and output gradients.  The number of paths and the weight width
come from the caller.

Workloads (the pages quote SevenNet-l3i5 at 4K atoms and MD up to 28K atoms in
the FlashTP summary's "Key results" and "Measured effects" table, and TP
microbenchmarks over l_max 1-5 in its "Experimental setup"; these synthetic
graphs stand in for those systems, whose datasets and weights are not used):

  tiny  16 atoms uniform in a 6 A cube, no periodic boundary, cutoff 4 A,
        4x0e+4x1o, SH l<=1, fp64, W ~ N(0,1)
  c1k   1024 atoms, density 0.1/A^3, periodic, cutoff 4.5 A,
        32x0e+32x1o+32x2e, SH l<=2, fp32
  c4k   4096 atoms, density 0.1/A^3, periodic, cutoff 5 A,
        32x0e+32x1o+32x2e+32x3o, SH l<=3, fp32 (SevenNet-l3i5-shaped)
  c2k   2048 atoms, density 0.1/A^3, periodic, cutoff 5 A,
        16 channels each of l=0..4 alternating parity, SH l<=4, fp64
  c28k  28000 atoms, density 0.1/A^3, periodic, cutoff 5 A,
        64x0e+64x1o+64x2e+64x3o, SH l<=3, fp32

SO(2) convolution shapes on the same graphs (SO2_SHAPES: degree bound L and
channels C, every l = 0..L present with C channels): tiny L=1 C=16, c1k L=2
C=32, c4k L=3 C=32, c2k L=3 C=16, c28k L=3 C=32; x and G N(0,1), the map
weights N(0,1)/sqrt(2 C (L+1)), fp32, from their own seeded stream.

Edges are ordered pairs (i != j) closer than the cutoff (minimum image when
periodic), src = j (neighbour), dst = i (centre), edge vector
r = pos[src] - pos[dst]; they are emitted dst-major, src ascending.  x and G
are N(0,1); W is N(0,1)/sqrt(n_paths) (tiny: N(0,1)).  Seeds:
numpy SeedSequence([2026, k]) for workload k = 1..5, draw order positions,
x, W, G.
"""

from __future__ import annotations

import re
from dataclasses import dataclass
from math import factorial, sqrt
from typing import Optional

import numpy as np
from scipy.spatial import cKDTree


@dataclass(frozen=True)
class Workload:
    key: int
    name: str
    n_atoms: int
    cutoff: float
    irreps_in: str
    sh_lmax: int
    irreps_out: str
    dtype: str            # "f32" or "f64"
    density: Optional[float] = None   # periodic cubic box of side (N/density)^(1/3)
    cube: Optional[float] = None      # non-periodic cube of this side
    scale_weights: bool = True

    @property
    def periodic(self) -> bool:
        return self.density is not None

    @property
    def box(self) -> float:
        return (self.n_atoms / self.density) ** (1.0 / 3.0) if self.periodic else float(self.cube)

    @property
    def np_dtype(self):
        return np.float32 if self.dtype == "f32" else np.float64


WORKLOADS = {
    "tiny": Workload(1, "tiny", 16, 4.0, "4x0e+4x1o", 1, "4x0e+4x1o", "f64", cube=6.0, scale_weights=False),
    "c1k": Workload(2, "c1k", 1024, 4.5, "32x0e+32x1o+32x2e", 2, "32x0e+32x1o+32x2e", "f32", density=0.1),
    "c4k": Workload(3, "c4k", 4096, 5.0, "32x0e+32x1o+32x2e+32x3o", 3, "32x0e+32x1o+32x2e+32x3o", "f32",
                    density=0.1),
    "c2k": Workload(4, "c2k", 2048, 5.0, "16x0e+16x1o+16x2e+16x3o+16x4e", 4, "16x0e+16x1o+16x2e+16x3o+16x4e",
                    "f64", density=0.1),
    "c28k": Workload(5, "c28k", 28000, 5.0, "64x0e+64x1o+64x2e+64x3o", 3, "64x0e+64x1o+64x2e+64x3o", "f32",
                     density=0.1),
}


SO2_SHAPES = {"tiny": (1, 16), "c1k": (2, 32), "c4k": (3, 32), "c2k": (3, 16), "c28k": (3, 32)}


def rng_for(key: int, stream: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([2026, key] + ([stream] if stream else [])))


def neighbour_list(pos: np.ndarray, cutoff: float, box: Optional[float]):
    """Ordered pairs closer than cutoff; returns (src, dst, vec) dst-major, src ascending."""
    n = pos.shape[0]
    if box is not None:
        tree = cKDTree(np.mod(pos, box), boxsize=box)
    else:
        tree = cKDTree(pos)
    pairs = tree.query_pairs(cutoff, output_type="ndarray")
    if pairs.size == 0:
        z = np.zeros(0, dtype=np.int64)
        return z, z, np.zeros((0, 3))
    a, b = pairs[:, 0], pairs[:, 1]
    dst = np.concatenate([a, b])
    src = np.concatenate([b, a])
    vec = pos[src] - pos[dst]
    if box is not None:
        vec = vec - box * np.round(vec / box)
    d = np.linalg.norm(vec, axis=1)
    keep = (d < cutoff) & (d > 0)
    src, dst, vec = src[keep], dst[keep], vec[keep]
    order = np.lexsort((src, dst))
    assert n == 0 or dst.max(initial=0) < n
    return src[order], dst[order], vec[order]


def real_sh(lmax: int, vec: np.ndarray) -> np.ndarray:
    """Real spherical harmonics, component normalisation (|Y_l|^2 = 2l+1).

    Built from the Cartesian form: for a unit vector (x, y, z),
      Y_l^0  = sqrt(2l+1) Q_l^0(z)
      Y_l^m  = sqrt(2l+1) sqrt(2 (l-m)!/(l+m)!) Q_l^m(z) Re (x + i y)^m   (m > 0)
      Y_l^-m = sqrt(2l+1) sqrt(2 (l-m)!/(l+m)!) Q_l^m(z) Im (x + i y)^m
    with Q_l^m = P_l^m / (1 - z^2)^(m/2) from the associated-Legendre recurrence
    without the Condon-Shortley sign.  Column of (l, m) is l*l + l + m.
    """
    vec = np.asarray(vec, dtype=np.float64)
    r = np.linalg.norm(vec, axis=-1, keepdims=True)
    u = vec / r
    x, y, z = u[..., 0], u[..., 1], u[..., 2]
    out = np.zeros(vec.shape[:-1] + ((lmax + 1) ** 2,))
    Q = {}
    for m in range(lmax + 1):
        dfact = 1.0
        for k in range(1, 2 * m, 2):
            dfact *= k
        Q[(m, m)] = np.full_like(z, dfact)
        if m + 1 <= lmax:
            Q[(m + 1, m)] = (2 * m + 1) * z * Q[(m, m)]
        for l in range(m + 2, lmax + 1):
            Q[(l, m)] = ((2 * l - 1) * z * Q[(l - 1, m)] - (l + m - 1) * Q[(l - 2, m)]) / (l - m)
    cplx = x + 1j * y
    powers = [np.ones_like(cplx)]
    for m in range(1, lmax + 1):
        powers.append(powers[-1] * cplx)
    for l in range(lmax + 1):
        base = l * l + l
        out[..., base] = sqrt(2 * l + 1) * Q[(l, 0)]
        for m in range(1, l + 1):
            nrm = sqrt(2 * l + 1) * sqrt(2.0 * factorial(l - m) / factorial(l + m))
            out[..., base + m] = nrm * Q[(l, m)] * powers[m].real
            out[..., base - m] = nrm * Q[(l, m)] * powers[m].imag
    return out


def positions(w: Workload, rng: np.random.Generator) -> np.ndarray:
    return rng.uniform(0.0, w.box, size=(w.n_atoms, 3))


def dim_of(irreps: str) -> int:
    """Row width of a feature vector for an irreps string (sum of mul*(2l+1))."""
    total = 0
    for term in irreps.split("+"):
        m = re.fullmatch(r"\s*(?:(\d+)\s*x\s*)?(\d+)\s*[eo]\s*", term)
        if m is None:
            raise ValueError(f"bad irreps term {term!r}")
        total += int(m.group(1) or 1) * (2 * int(m.group(2)) + 1)
    return total


def make_graph(w: Workload):
    """Positions and neighbour list; returns dict(pos, src, dst, vec, Y)."""
    rng = rng_for(w.key)
    pos = positions(w, rng)
    src, dst, vec = neighbour_list(pos, w.cutoff, w.box if w.periodic else None)
    return dict(pos=pos, src=src.astype(np.int32), dst=dst.astype(np.int32), vec=vec, rng=rng)


def make_inputs(w: Workload, n_paths: int, weight_numel: int):
    """All inputs of one forward+backward in the workload's dtype (numpy).

    Returns dict with n_nodes, src, dst (int32), Y [E, (L+1)^2], x [N, D_in],
    W [E, weight_numel], G [N, D_out], and pos / vec for reference.
    """
    g = make_graph(w)
    rng = g.pop("rng")
    dt = w.np_dtype
    E = g["src"].shape[0]
    d_in, d_out = dim_of(w.irreps_in), dim_of(w.irreps_out)
    Y = real_sh(w.sh_lmax, g["vec"]).astype(dt) if E else np.zeros((0, (w.sh_lmax + 1) ** 2), dtype=dt)
    x = rng.standard_normal((w.n_atoms, d_in), dtype=dt)
    W = rng.standard_normal((E, weight_numel), dtype=dt)
    if w.scale_weights and n_paths > 0:
        W *= dt(1.0 / sqrt(n_paths))
    G = rng.standard_normal((w.n_atoms, d_out), dtype=dt)
    g.update(n_nodes=w.n_atoms, Y=Y, x=x, W=W, G=G)
    return g


def make_cotangents(w: Workload, n_edges: int, weight_numel: int):
    """Cotangents of the backward's outputs, the double backward's extra inputs:
    ggx [N, D_in], ggY [E, (L+1)^2], ggW [E, weight_numel], standard normal in
    the workload's dtype, from their own seeded stream (make_inputs' draws are
    unchanged by it)."""
    rng = rng_for(w.key, stream=2)
    dt = w.np_dtype
    ggx = rng.standard_normal((w.n_atoms, dim_of(w.irreps_in)), dtype=dt)
    ggY = rng.standard_normal((n_edges, (w.sh_lmax + 1) ** 2), dtype=dt)
    ggW = rng.standard_normal((n_edges, weight_numel), dtype=dt)
    return dict(ggx=ggx, ggY=ggY, ggW=ggW)


def random_rotation(rng: np.random.Generator) -> np.ndarray:
    """Uniform random proper rotation (QR of a Gaussian matrix, sign-fixed)."""
    q, r = np.linalg.qr(rng.standard_normal((3, 3)))
    q = q * np.sign(np.diag(r))
    if np.linalg.det(q) < 0:
        q[:, 0] = -q[:, 0]
    return q


def make_so2_inputs(w: Workload, weight_numel: int):
    """Inputs of one SO(2)-convolution forward+backward on workload w's graph
    (fp32 numpy): dict(n_nodes, src, dst, vec, lmax, channels, x, weights, G)
    with x, G [N, C (L+1)^2] and weights [weight_numel] (the width comes from
    the caller)."""
    lmax, C = SO2_SHAPES[w.name]
    g = make_graph(w)
    g.pop("rng")
    rng = rng_for(w.key, stream=3)
    d = C * (lmax + 1) ** 2
    x = rng.standard_normal((w.n_atoms, d), dtype=np.float32)
    weights = rng.standard_normal(weight_numel, dtype=np.float32) * np.float32(1.0 / sqrt(2.0 * C * (lmax + 1)))
    G = rng.standard_normal((w.n_atoms, d), dtype=np.float32)
    g.update(n_nodes=w.n_atoms, lmax=lmax, channels=C, x=x, weights=weights, G=G)
    return g

