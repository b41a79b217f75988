"""Clebsch-Gordan coefficients, complex and real basis (oracle; test infrastructure).

The FlashTP summary ("Problem", "Approach") says the tensor product runs over a
sparse Clebsch-Gordan coefficient matrix; the pages do not print it, so the
textbook definitions are written out:

* Complex CG <l1 m1 l2 m2 | l3 m3> by Racah's closed form with the
  Condon-Shortley phase, evaluated exactly with Python integers/fractions and
  rounded once to fp64.
* Real basis: U^l maps complex components (columns, mu = -l..l) to real ones
  (rows, m = -l..l):
      m = 0 :  U[0, 0] = 1
      m > 0 :  U[m, m] = (-1)^m / sqrt2,   U[m, -m] = 1 / sqrt2
      m < 0 :  U[m, m] = i / sqrt2,        U[m, -m] = -i (-1)^|m| / sqrt2
  and  C_real[m1,m2,m3] = sum U1[m1,a] U2[m2,b] conj(U3[m3,c]) <l1 a l2 b|l3 c>.
  The sum is real for even l1+l2+l3 and purely imaginary for odd l1+l2+l3;
  the odd case takes the imaginary part (an overall sign per path that keeps
  the coupling equivariant).
"""

from __future__ import annotations

from fractions import Fraction
from functools import lru_cache
from math import factorial, sqrt

import numpy as np


def _triangle(l1: int, l2: int, l3: int) -> bool:
    return abs(l1 - l2) <= l3 <= l1 + l2


def cg_complex_squared(l1: int, m1: int, l2: int, m2: int, l3: int, m3: int):
    """Exact (sign, CG^2 as Fraction) of <l1 m1 l2 m2 | l3 m3> by Racah's formula."""
    if m3 != m1 + m2 or not _triangle(l1, l2, l3):
        return 0, Fraction(0)
    if abs(m1) > l1 or abs(m2) > l2 or abs(m3) > l3:
        return 0, Fraction(0)
    f = factorial
    pref = Fraction((2 * l3 + 1) * f(l3 + l1 - l2) * f(l3 - l1 + l2) * f(l1 + l2 - l3), f(l1 + l2 + l3 + 1))
    pref *= f(l3 + m3) * f(l3 - m3) * f(l1 - m1) * f(l1 + m1) * f(l2 - m2) * f(l2 + m2)
    s = Fraction(0)
    for k in range(0, l1 + l2 + l3 + 1):
        args = (k, l1 + l2 - l3 - k, l1 - m1 - k, l2 + m2 - k, l3 - l2 + m1 + k, l3 - l1 - m2 + k)
        if min(args) < 0:
            continue
        den = 1
        for a in args:
            den *= f(a)
        s += Fraction((-1) ** k, den)
    if s == 0:
        return 0, Fraction(0)
    return (1 if s > 0 else -1), pref * s * s


def cg_complex(l1: int, m1: int, l2: int, m2: int, l3: int, m3: int) -> float:
    """<l1 m1 l2 m2 | l3 m3> as fp64 (Condon-Shortley phase)."""
    sign, sq = cg_complex_squared(l1, m1, l2, m2, l3, m3)
    if sign == 0:
        return 0.0
    return sign * sqrt(float(sq))


def real_basis_U(l: int) -> np.ndarray:
    """U^l, shape (2l+1, 2l+1), rows real m = -l..l, columns complex mu = -l..l."""
    n = 2 * l + 1
    U = np.zeros((n, n), dtype=np.complex128)
    r = 1.0 / sqrt(2.0)
    for m in range(-l, l + 1):
        row = m + l
        if m == 0:
            U[row, l] = 1.0
        elif m > 0:
            U[row, m + l] = (-1) ** m * r
            U[row, -m + l] = r
        else:
            k = -m
            U[row, -k + l] = 1j * r
            U[row, k + l] = -1j * (-1) ** k * r
    return U


@lru_cache(maxsize=None)
def _cg_complex_dense(l1: int, l2: int, l3: int) -> np.ndarray:
    T = np.zeros((2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1))
    for m1 in range(-l1, l1 + 1):
        for m2 in range(-l2, l2 + 1):
            m3 = m1 + m2
            if abs(m3) <= l3:
                T[m1 + l1, m2 + l2, m3 + l3] = cg_complex(l1, m1, l2, m2, l3, m3)
    return T


@lru_cache(maxsize=None)
def cg_real(l1: int, l2: int, l3: int) -> np.ndarray:
    """Dense real-basis CG tensor C[m1, m2, m3] (indices 0..2l, i.e. m + l)."""
    if not _triangle(l1, l2, l3):
        raise ValueError(f"({l1},{l2},{l3}) violates the triangle rule")
    T = _cg_complex_dense(l1, l2, l3).astype(np.complex128)
    U1, U2, U3 = real_basis_U(l1), real_basis_U(l2), real_basis_U(l3)
    C = np.einsum("ia,jb,kc,abc->ijk", U1, U2, U3.conj(), T)
    if (l1 + l2 + l3) % 2 == 0:
        out = C.real.copy()
    else:
        out = C.imag.copy()
    out[np.abs(out) < 1e-14] = 0.0
    out.setflags(write=False)
    return out
