"""Edge spherical harmonics with their gradient, and the position gradient
(oracle; test infrastructure).

The step upstream of the convolution: Y_e = Y(r_e / |r_e|) from the edge
vector r_e = pos[src] - pos[dst] (plus a constant periodic shift), and the
chain rule back from dL/dY_e to dL/dr_e and on to the atom positions, which
gives forces as -dE/dpos.  (The LunaTP and TrimSO(2) abstracts frame the
operator within force-field training; the pages give no formula for this
step, so it is written out from the definition of the harmonics in sh.py.)

Each block Y_l restricted to the unit sphere is a homogeneous polynomial of
degree l in (x, y, z).  Its coefficients in the monomial basis x^a y^b z^c
(a + b + c = l) are found once per l by a least-squares fit to sh_real at
random points; the fit is exact up to rounding because the restriction of
degree-l homogeneous polynomials to the sphere is injective and contains the
degree-l harmonics.  With p_lm that polynomial and r_hat = r / |r|,

    dY_lm / dr = ( grad p_lm(r_hat) - l * p_lm(r_hat) * r_hat ) / |r|

(the gradient of p_lm(r / |r|); r_hat . grad p_lm = l p_lm for a homogeneous
polynomial).  A zero vector has no direction: Y = (1, 0, ..., 0) and a zero
gradient there, by convention.
"""

from __future__ import annotations

from functools import lru_cache

import numpy as np

from .sh import sh_real


def _monomials(l: int):
    return [(a, b, l - a - b) for a in range(l, -1, -1) for b in range(l - a, -1, -1)]


@lru_cache(maxsize=None)
def sh_poly_coeffs(l: int) -> np.ndarray:
    """C [2l+1, n_mono]: Y_l(r_hat) = C @ [x^a y^b z^c for (a, b, c) in _monomials(l)]."""
    mons = _monomials(l)
    rng = np.random.default_rng(1000 + l)
    pts = rng.standard_normal((8 * len(mons) + 16, 3))
    pts /= np.linalg.norm(pts, axis=1, keepdims=True)
    A = np.stack([pts[:, 0] ** a * pts[:, 1] ** b * pts[:, 2] ** c for a, b, c in mons], axis=1)
    B = sh_real(l, pts)[:, l * l:]
    C, *_ = np.linalg.lstsq(A, B, rcond=None)
    resid = np.max(np.abs(A @ C - B))
    if resid > 1e-11:
        raise AssertionError(f"l={l}: harmonic polynomial fit residual {resid}")
    return C.T.copy()


def sh_and_jacobian(lmax: int, vec):
    """Y [E, (lmax+1)^2] and J [E, (lmax+1)^2, 3] = dY / dvec."""
    vec = np.asarray(vec, dtype=np.float64)
    E = vec.shape[0]
    D = (lmax + 1) ** 2
    r = np.linalg.norm(vec, axis=1)
    ok = r > 0
    rh = np.zeros_like(vec)
    rh[ok] = vec[ok] / r[ok, None]
    Y = np.zeros((E, D))
    J = np.zeros((E, D, 3))
    x, y, z = rh[:, 0], rh[:, 1], rh[:, 2]
    for l in range(lmax + 1):
        C = sh_poly_coeffs(l)
        mons = _monomials(l)
        val = np.stack([x ** a * y ** b * z ** c for a, b, c in mons], axis=1)            # [E, M]
        grad = np.zeros((E, len(mons), 3))
        for k, (a, b, c) in enumerate(mons):
            if a:
                grad[:, k, 0] = a * x ** (a - 1) * y ** b * z ** c
            if b:
                grad[:, k, 1] = b * x ** a * y ** (b - 1) * z ** c
            if c:
                grad[:, k, 2] = c * x ** a * y ** b * z ** (c - 1)
        p = val @ C.T                                                                    # [E, 2l+1]
        gp = np.einsum("mk,ekd->emd", C, grad)                                           # [E, 2l+1, 3]
        Jl = (gp - l * p[:, :, None] * rh[:, None, :]) / np.where(ok, r, 1.0)[:, None, None]
        Y[:, l * l:(l + 1) ** 2] = p
        J[:, l * l:(l + 1) ** 2] = Jl
    Y[~ok] = 0.0
    Y[~ok, 0] = 1.0
    J[~ok] = 0.0
    return Y, J


def sh_edges(lmax: int, vec) -> np.ndarray:
    """Y [E, (lmax+1)^2] of the edge vectors (zero vector -> (1, 0, ..., 0))."""
    return sh_and_jacobian(lmax, vec)[0]


def sh_backward(lmax: int, vec, grad_Y) -> np.ndarray:
    """grad_vec [E, 3] = sum_lm grad_Y[e, lm] dY_lm / dvec_e."""
    _, J = sh_and_jacobian(lmax, vec)
    return np.einsum("ed,edk->ek", np.asarray(grad_Y, dtype=np.float64), J)


def positions_backward(grad_vec, src, dst, n_nodes: int) -> np.ndarray:
    """grad_pos [N, 3] for r_e = pos[src] - pos[dst] (+ a constant shift):
    each edge adds grad_vec[e] to its source and subtracts it from its destination."""
    g = np.asarray(grad_vec, dtype=np.float64)
    out = np.zeros((n_nodes, 3))
    np.add.at(out, np.asarray(src, dtype=np.int64), g)
    np.add.at(out, np.asarray(dst, dtype=np.int64), -g)
    return out


__all__ = ["sh_poly_coeffs", "sh_and_jacobian", "sh_edges", "sh_backward", "positions_backward"]
