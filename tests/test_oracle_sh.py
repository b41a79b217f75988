"""Pins for the oracle's real spherical harmonics and the input generator's (CPU only)."""

import numpy as np
import pytest
from scipy import special

import workloads
from oracle.sh import sh_real


def unit(rng, n):
    v = rng.standard_normal((n, 3))
    return v / np.linalg.norm(v, axis=1, keepdims=True)


def test_low_orders_closed_form():
    rng = np.random.default_rng(1)
    v = unit(rng, 50)
    Y = sh_real(1, v)
    np.testing.assert_allclose(Y[:, 0], 1.0, atol=1e-15)
    np.testing.assert_allclose(Y[:, 1:4], np.sqrt(3) * v[:, [1, 2, 0]], atol=1e-14)


@pytest.mark.parametrize("lmax", [0, 2, 4, 6])
def test_component_norm_and_pole(lmax):
    rng = np.random.default_rng(2)
    Y = sh_real(lmax, unit(rng, 40))
    for l in range(lmax + 1):
        np.testing.assert_allclose((Y[:, l * l:(l + 1) ** 2] ** 2).sum(1), 2 * l + 1, rtol=1e-13)
    z = sh_real(lmax, np.array([[0.0, 0.0, 1.0]]))[0]
    for l in range(lmax + 1):
        e = np.zeros(2 * l + 1)
        e[l] = np.sqrt(2 * l + 1)
        np.testing.assert_allclose(z[l * l:(l + 1) ** 2], e, atol=1e-14)


@pytest.mark.parametrize("lmax", [3, 4])
def test_addition_theorem(lmax):
    """sum_m Y_lm(a) Y_lm(b) = (2l+1) P_l(a.b) in component normalisation."""
    rng = np.random.default_rng(3)
    a, b = unit(rng, 30), unit(rng, 30)
    Ya, Yb = sh_real(lmax, a), sh_real(lmax, b)
    c = (a * b).sum(1)
    for l in range(lmax + 1):
        s = (Ya[:, l * l:(l + 1) ** 2] * Yb[:, l * l:(l + 1) ** 2]).sum(1)
        np.testing.assert_allclose(s, (2 * l + 1) * special.eval_legendre(l, c), atol=1e-12)


def test_orthonormal_by_quadrature():
    xg, wg = np.polynomial.legendre.leggauss(12)
    nphi = 24
    phi = (np.arange(nphi) + 0.5) * 2 * np.pi / nphi
    ct, ph = np.meshgrid(xg, phi, indexing="ij")
    st = np.sqrt(1 - ct**2)
    pts = np.stack([st * np.cos(ph), st * np.sin(ph), ct], -1).reshape(-1, 3)
    w = (wg[:, None] * np.full(nphi, 2 * np.pi / nphi)).ravel()
    Y = sh_real(4, pts, normalization="integral")
    np.testing.assert_allclose(Y.T @ (w[:, None] * Y), np.eye(25), atol=1e-13)


@pytest.mark.parametrize("lmax", [1, 3, 4])
def test_generator_sh_equals_oracle_sh(lmax):
    """The input generator's Cartesian recurrence and the oracle's scipy-based SH agree."""
    rng = np.random.default_rng(4)
    v = rng.standard_normal((200, 3)) * 3.0
    np.testing.assert_allclose(workloads.real_sh(lmax, v), sh_real(lmax, v), atol=1e-13)


def test_generator_graphs_match_brute_force():
    for name in ("tiny", "c1k"):
        w = workloads.WORKLOADS[name]
        g = workloads.make_graph(w)
        pos = g["pos"]
        d = pos[None, :, :] - pos[:, None, :]   # d[i, j] = pos[j] - pos[i]
        if w.periodic:
            d -= w.box * np.round(d / w.box)
        r = np.linalg.norm(d, axis=-1)
        np.fill_diagonal(r, np.inf)
        dst, src = np.nonzero(r < w.cutoff)
        np.testing.assert_array_equal(g["dst"], dst)
        np.testing.assert_array_equal(g["src"], src)
        np.testing.assert_allclose(g["vec"], d[dst, src], atol=1e-12)
