"""Pins for the oracle's Clebsch-Gordan tables (CPU only).

Each check uses mathematics the oracle does not itself use: sympy's CG routine,
a printed textbook table, unitarity, closed-form special values, and the Gaunt
integral of three real spherical harmonics evaluated by exact quadrature.
"""

import itertools
import os
from math import sqrt

import numpy as np
import pytest

from oracle.cg import cg_complex, cg_real, real_basis_U
from oracle.sh import sh_real

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def triples(lmax):
    for l1, l2 in itertools.product(range(lmax + 1), repeat=2):
        for l3 in range(abs(l1 - l2), min(l1 + l2, lmax) + 1):
            yield l1, l2, l3


def test_textbook_table_1x1():
    path = os.path.join(GOLDEN, "cg_textbook_1x1.txt")
    rows = [ln.split() for ln in open(path) if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 19
    for m1, m2, J, M, sign, num, den in (map(int, r) for r in rows):
        expect = sign * sqrt(num / den)
        assert cg_complex(1, m1, 1, m2, J, M) == pytest.approx(expect, abs=1e-15), (m1, m2, J, M)


def test_racah_matches_sympy():
    sympy_cg = pytest.importorskip("sympy.physics.quantum.cg")
    S = pytest.importorskip("sympy")
    rng = np.random.default_rng(7)
    cases = []
    for l1, l2, l3 in triples(3):
        for m1 in range(-l1, l1 + 1):
            for m2 in range(-l2, l2 + 1):
                if abs(m1 + m2) <= l3:
                    cases.append((l1, m1, l2, m2, l3, m1 + m2))
    # all l <= 2 cases, plus a random sample of the l = 3, 4 ones
    small = [c for c in cases if max(c[0], c[2], c[4]) <= 2]
    big = [c for c in cases if max(c[0], c[2], c[4]) > 2]
    extra = []
    for l1, l2, l3 in triples(4):
        if max(l1, l2, l3) == 4:
            m1 = int(rng.integers(-l1, l1 + 1))
            for m2 in range(-l2, l2 + 1):
                if abs(m1 + m2) <= l3:
                    extra.append((l1, m1, l2, m2, l3, m1 + m2))
    pick = small + [big[i] for i in rng.choice(len(big), 120, replace=False)] + extra[::3]
    for c in pick:
        ref = float(S.N(sympy_cg.CG(*c).doit(), 30))
        assert cg_complex(*c) == pytest.approx(ref, abs=2e-15), c


def test_complex_cg_orthogonality_and_completeness():
    for l1, l2 in itertools.product(range(4), repeat=2):
        rows = []
        labels = []
        for l3 in range(abs(l1 - l2), l1 + l2 + 1):
            for m3 in range(-l3, l3 + 1):
                v = np.zeros((2 * l1 + 1, 2 * l2 + 1))
                for m1 in range(-l1, l1 + 1):
                    m2 = m3 - m1
                    if abs(m2) <= l2:
                        v[m1 + l1, m2 + l2] = cg_complex(l1, m1, l2, m2, l3, m3)
                rows.append(v.ravel())
                labels.append((l3, m3))
        M = np.array(rows)
        n = (2 * l1 + 1) * (2 * l2 + 1)
        assert M.shape == (n, n)
        np.testing.assert_allclose(M @ M.T, np.eye(n), atol=1e-14)
        np.testing.assert_allclose(M.T @ M, np.eye(n), atol=1e-14)


@pytest.mark.parametrize("l", range(5))
def test_complex_cg_special_values(l):
    for m in range(-l, l + 1):
        assert cg_complex(l, m, 0, 0, l, m) == pytest.approx(1.0, abs=1e-15)
        assert cg_complex(0, 0, l, m, l, m) == pytest.approx(1.0, abs=1e-15)
        assert cg_complex(l, m, l, -m, 0, 0) == pytest.approx((-1) ** (l - m) / sqrt(2 * l + 1), abs=1e-15)
    for l2 in range(5):
        assert cg_complex(l, l, l2, l2, l + l2, l + l2) == pytest.approx(1.0, abs=1e-15)
    assert cg_complex(l, 0, l, 0, 1, 0) == 0.0  # odd l1+l2+l3 with all m = 0 vanishes
    assert cg_complex(l, 1 if l else 0, 1, 0, l, 0) == 0.0  # m selection rule


def test_real_basis_is_unitary():
    for l in range(6):
        U = real_basis_U(l)
        np.testing.assert_allclose(U @ U.conj().T, np.eye(2 * l + 1), atol=1e-15)


@pytest.mark.parametrize("l1,l2,l3", list(triples(4)))
def test_real_cg_is_an_isometry(l1, l2, l3):
    C = cg_real(l1, l2, l3).reshape(-1, 2 * l3 + 1)
    np.testing.assert_allclose(C.T @ C, np.eye(2 * l3 + 1), atol=1e-14)


def _sphere_quadrature(nt=24, nphi=48):
    """Gauss-Legendre in cos(theta) x uniform phi: exact for SH products of degree < min(2nt, nphi)."""
    xg, wg = np.polynomial.legendre.leggauss(nt)
    phi = (np.arange(nphi) + 0.5) * 2 * np.pi / nphi
    ct, ph = np.meshgrid(xg, phi, indexing="ij")
    st = np.sqrt(1 - ct**2)
    pts = np.stack([st * np.cos(ph), st * np.sin(ph), ct], -1).reshape(-1, 3)
    w = (wg[:, None] * np.full(nphi, 2 * np.pi / nphi)[None, :]).ravel()
    return pts, w


@pytest.mark.parametrize("l1,l2,l3", [t for t in triples(4) if sum(t) % 2 == 0])
def test_real_cg_matches_gaunt_integral(l1, l2, l3):
    """int Y_l1m1 Y_l2m2 Y_l3m3 dOmega = sqrt((2l1+1)(2l2+1)/(4pi(2l3+1))) <l1 0 l2 0|l3 0> C_real."""
    pts, w = _sphere_quadrature()
    L = max(l1, l2, l3)
    Y = sh_real(L, pts, normalization="integral")
    b = lambda l: Y[:, l * l:(l + 1) ** 2]  # noqa: E731
    gaunt = np.einsum("q,qi,qj,qk->ijk", w, b(l1), b(l2), b(l3))
    pref = sqrt((2 * l1 + 1) * (2 * l2 + 1) / (4 * np.pi * (2 * l3 + 1))) * cg_complex(l1, 0, l2, 0, l3, 0)
    np.testing.assert_allclose(gaunt, pref * cg_real(l1, l2, l3), atol=1e-13)


def test_real_cg_known_patterns():
    # l x 0 -> l and 0 x l -> l are identities
    for l in range(5):
        np.testing.assert_allclose(cg_real(l, 0, l)[:, 0, :], np.eye(2 * l + 1), atol=1e-15)
        np.testing.assert_allclose(cg_real(0, l, l)[0], np.eye(2 * l + 1), atol=1e-15)
    # 1 x 1 -> 0 is -1/sqrt(3) times the identity (a dot product)
    np.testing.assert_allclose(cg_real(1, 1, 0)[:, :, 0], -np.eye(3) / sqrt(3), atol=1e-15)
    # l x l -> 0 in general: one coefficient (-1)^l / sqrt(2l+1) on the diagonal,
    # from <l m l -m|0 0> = (-1)^(l-m) / sqrt(2l+1) and the unitarity of U
    for l in range(5):
        np.testing.assert_allclose(cg_real(l, l, 0)[:, :, 0], (-1) ** l * np.eye(2 * l + 1) / sqrt(2 * l + 1),
                                   atol=1e-15)
    # 1 x 1 -> 1 (odd sum) is a cross product: components ordered (y, z, x)
    C = cg_real(1, 1, 1)
    rng = np.random.default_rng(0)
    a, b = rng.standard_normal(3), rng.standard_normal(3)
    perm = [1, 2, 0]  # real m = -1, 0, 1  <->  y, z, x
    z = np.einsum("i,j,ijk->k", a[perm], b[perm], C)
    cross = np.cross(a, b)[perm]
    ratio = z / cross
    np.testing.assert_allclose(np.abs(ratio), 1 / sqrt(2), rtol=1e-13)
    assert np.all(np.sign(ratio) == np.sign(ratio[0]))


def test_real_cg_nonzero_counts():
    """Nonzeros of the real tables for the l<=3 paths with even l1+l2+l3 (353 over the 23 paths)."""
    even = [t for t in triples(3) if sum(t) % 2 == 0]
    assert len(even) == 23
    assert sum(int(np.count_nonzero(cg_real(*t))) for t in even) == 353
