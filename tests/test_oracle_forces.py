"""Pins for the oracle's edge harmonics, their gradient and the position gradient (CPU only).

Checked against things the oracle does not itself use for the gradient:
central finite differences of the (separately pinned) sh_real, the
tangency of the gradient (Y depends on the direction only), homogeneity
of degree -1, the closed form of the l = 1 block, rotation covariance with
Wigner-D matrices fitted from the harmonics, and finite differences of a
whole energy <G, out> in the atom positions through the pinned convolution.
"""

import numpy as np
import pytest

from oracle import (TPProblem, positions_backward, sh_and_jacobian, sh_backward, sh_edges, sh_real,
                    tp_backward, tp_forward)

from test_oracle_tp import fitted_D


@pytest.mark.parametrize("lmax", [0, 1, 2, 3, 4])
def test_values_match_the_pinned_harmonics(lmax):
    v = np.random.default_rng(40 + lmax).standard_normal((60, 3)) * 3.0
    Y, _ = sh_and_jacobian(lmax, v)
    np.testing.assert_allclose(Y, sh_real(lmax, v), atol=1e-13)


@pytest.mark.parametrize("lmax", [1, 2, 3, 4])
def test_jacobian_by_central_differences(lmax):
    rng = np.random.default_rng(50 + lmax)
    v = rng.standard_normal((40, 3)) * 2.0
    _, J = sh_and_jacobian(lmax, v)
    h = 1e-5
    for _ in range(3):
        d = rng.standard_normal((40, 3))
        fd = (sh_real(lmax, v + h * d) - sh_real(lmax, v - h * d)) / (2 * h)
        np.testing.assert_allclose(np.einsum("edk,ek->ed", J, d), fd, atol=5e-8)


def test_tangency_homogeneity_and_l1_closed_form():
    rng = np.random.default_rng(60)
    v = rng.standard_normal((30, 3)) * 1.7
    _, J = sh_and_jacobian(4, v)
    # Y depends on the direction only: no radial derivative
    np.testing.assert_allclose(np.einsum("edk,ek->ed", J, v), 0.0, atol=1e-12)
    # degree -1 in |r|
    _, J2 = sh_and_jacobian(4, 2.5 * v)
    np.testing.assert_allclose(J2, J / 2.5, atol=1e-13)
    # Y_1 = sqrt(3) (y, z, x) / |r|  =>  dY_1/dr = sqrt(3) P (I - r_hat r_hat^T) / |r|
    r = np.linalg.norm(v, axis=1)
    rh = v / r[:, None]
    proj = (np.eye(3)[None] - rh[:, :, None] * rh[:, None, :]) / r[:, None, None]
    perm = [1, 2, 0]
    np.testing.assert_allclose(J[:, 1:4], np.sqrt(3.0) * proj[:, perm, :], atol=1e-13)


def test_rotation_covariance():
    rng = np.random.default_rng(61)
    v = rng.standard_normal((25, 3))
    q, rr = np.linalg.qr(rng.standard_normal((3, 3)))
    R = q * np.sign(np.diag(rr))
    if np.linalg.det(R) < 0:
        R[:, 0] *= -1
    _, J = sh_and_jacobian(4, v)
    _, Jr = sh_and_jacobian(4, v @ R.T)
    for l in range(5):
        D = fitted_D(l, R, rng)
        sl = slice(l * l, (l + 1) ** 2)
        # Y(R v) = D Y(v)  =>  J(R v) R = D J(v)
        np.testing.assert_allclose(np.einsum("edk,kj->edj", Jr[:, sl], R), np.einsum("mn,enk->emk", D, J[:, sl]),
                                   atol=1e-11)


def test_zero_vector_convention():
    v = np.array([[0.0, 0.0, 0.0], [1.0, 0.0, 0.0]])
    Y, J = sh_and_jacobian(3, v)
    assert Y[0, 0] == 1.0 and np.all(Y[0, 1:] == 0.0) and np.all(J[0] == 0.0)
    np.testing.assert_allclose(Y[1], sh_real(3, v[1:])[0], atol=1e-14)


def test_positions_backward_brute_force():
    rng = np.random.default_rng(62)
    n, E = 9, 40
    src, dst = rng.integers(0, n, E), rng.integers(0, n, E)
    g = rng.standard_normal((E, 3))
    ref = np.zeros((n, 3))
    for e in range(E):
        ref[src[e]] += g[e]
        ref[dst[e]] -= g[e]
    np.testing.assert_allclose(positions_backward(g, src, dst, n), ref, atol=1e-14)


@pytest.mark.parametrize("case", [("2x0e+2x1o", 1, "2x0e+2x1o"), ("1x0e+1x1o+1x2e+1x3o", 3, "1x0e+1x1o+1x2e+1x3o"),
                                  ("2x1o+2x2e", 4, "2x0e+2x1o+2x3o")])
def test_energy_gradient_in_positions(case):
    """E(pos) = <G, out(x, Y(pos[src] - pos[dst] + shift), W)>: the chain
    backward -> sh_backward -> positions_backward against central differences."""
    rng = np.random.default_rng(63)
    prob = TPProblem.build(*case)
    n = 7
    pairs = [(i, j) for i in range(n) for j in range(n) if i != j and rng.random() < 0.5]
    dst = np.array([p[0] for p in pairs])
    src = np.array([p[1] for p in pairs])
    E = len(src)
    pos = rng.standard_normal((n, 3)) * 2.0
    shift = rng.standard_normal((E, 3))          # periodic images: constant in pos
    x = rng.standard_normal((n, prob.dim_in))
    W = rng.standard_normal((E, prob.weight_numel))
    G = rng.standard_normal((n, prob.dim_out))

    def energy(p):
        Y = sh_edges(prob.sh_lmax, p[src] - p[dst] + shift)
        return np.vdot(G, tp_forward(prob, x, Y, W, src, dst, n))

    vec = pos[src] - pos[dst] + shift
    _, dY, _ = tp_backward(prob, x, sh_edges(prob.sh_lmax, vec), W, G, src, dst, n)
    grad = positions_backward(sh_backward(prob.sh_lmax, vec, dY), src, dst, n)
    h = 1e-5
    for _ in range(3):
        d = rng.standard_normal((n, 3))
        fd = (energy(pos + h * d) - energy(pos - h * d)) / (2 * h)
        assert fd == pytest.approx(np.vdot(grad, d), rel=1e-7, abs=1e-8)
