"""Real spherical harmonics (oracle; test infrastructure).

The convolution takes the edge's real spherical harmonics Y(r_ij) as an input.
The oracle builds them from scipy's complex spherical harmonics (Condon-Shortley
phase, orthonormal) through the same real basis U^l as the real CG table:

    Y_real_l(r) = sqrt(4 pi) * U^l  Y_complex_l(r)

The factor sqrt(4 pi) gives "component" normalisation, |Y_l(r)|^2 = 2l+1, so
Y_0 = 1 and Y_1 = sqrt(3) (y, z, x) for m = -1, 0, 1.  Row layout: (l, m) sits
at column l*l + l + m.
"""

from __future__ import annotations

import numpy as np
from scipy import special

from .cg import real_basis_U


def _angles(vec: np.ndarray):
    vec = np.asarray(vec, dtype=np.float64)
    r = np.linalg.norm(vec, axis=-1)
    if np.any(r == 0):
        raise ValueError("zero-length vector has no direction")
    z = np.clip(vec[..., 2] / r, -1.0, 1.0)
    theta = np.arccos(z)
    phi = np.arctan2(vec[..., 1], vec[..., 0])
    return theta, phi


def sh_complex(l: int, vec: np.ndarray) -> np.ndarray:
    """Orthonormal complex Y_l^mu(r_hat), shape (..., 2l+1), mu = -l..l."""
    theta, phi = _angles(vec)
    cols = [special.sph_harm_y(l, mu, theta, phi) for mu in range(-l, l + 1)]
    return np.stack(cols, axis=-1)


def sh_real(lmax: int, vec: np.ndarray, normalization: str = "component") -> np.ndarray:
    """Real SH for l = 0..lmax, shape (..., (lmax+1)^2)."""
    blocks = []
    for l in range(lmax + 1):
        yc = sh_complex(l, vec)
        yr = np.einsum("mk,...k->...m", real_basis_U(l), yc)
        if np.max(np.abs(yr.imag), initial=0.0) > 1e-12:
            raise AssertionError("real SH came out complex")
        blocks.append(yr.real)
    Y = np.concatenate(blocks, axis=-1)
    if normalization == "component":
        Y = Y * np.sqrt(4.0 * np.pi)
    elif normalization != "integral":
        raise ValueError(normalization)
    return Y
