"""Pins for the oracle's double backward (CPU only).

The double backward returns the gradients of
L2 = <a, dx> + <b, dY> + <c, dW> with respect to x, Y, W and G, where
(dx, dY, dW) is the backward of the convolution and (a, b, c) are the
cotangents of its three outputs.  It is pinned against the already pinned
forward and backward, never against its own formulas:

* finite differences of L2 computed through tp_backward -- L2 is linear in
  each of x, Y, W, G separately, so a central difference is exact up to
  rounding for any step;
* Euler's identity for functions linear in one argument, e.g. <gG, G> = L2;
* one cotangent at a time reduces every output to the forward or the backward
  evaluated with one argument replaced by that cotangent;
* rotation equivariance of all four outputs.
"""

import numpy as np
import pytest

from oracle import TPProblem, sh_real, tp_backward, tp_double_backward, tp_forward

from test_oracle_tp import CASES, apply_D, fitted_D, random_inputs, small_graph


def cotangents(rng, prob, n, E):
    a = rng.standard_normal((n, prob.dim_in))
    b = rng.standard_normal((E, prob.dim_sh))
    c = rng.standard_normal((E, prob.weight_numel))
    return a, b, c


def L2(prob, x, Y, W, G, a, b, c, src, dst, n):
    dx, dY, dW = tp_backward(prob, x, Y, W, G, src, dst, n)
    return np.vdot(a, dx) + np.vdot(b, dY) + np.vdot(c, dW)


@pytest.mark.parametrize("case", CASES)
def test_finite_differences_are_exact(case):
    rng = np.random.default_rng(21)
    prob = TPProblem.build(*case)
    n = 8
    src, dst = small_graph(rng, n=n, p=0.5)
    x, _, Y, W, G = random_inputs(rng, prob, n, len(src))
    a, b, c = cotangents(rng, prob, n, len(src))
    gx, gY, gW, gG = tp_double_backward(prob, x, Y, W, G, a, b, c, src, dst, n)
    args = dict(x=x, Y=Y, W=W, G=G)
    h = 0.61
    for name, grad in (("x", gx), ("Y", gY), ("W", gW), ("G", gG)):
        for _ in range(3):
            d = rng.standard_normal(args[name].shape)
            plus = dict(args, **{name: args[name] + h * d})
            minus = dict(args, **{name: args[name] - h * d})
            fd = (L2(prob, plus["x"], plus["Y"], plus["W"], plus["G"], a, b, c, src, dst, n)
                  - L2(prob, minus["x"], minus["Y"], minus["W"], minus["G"], a, b, c, src, dst, n)) / (2 * h)
            assert fd == pytest.approx(np.vdot(grad, d), rel=1e-10, abs=1e-10), name


@pytest.mark.parametrize("case", CASES)
def test_euler_identities(case):
    rng = np.random.default_rng(22)
    prob = TPProblem.build(*case)
    n = 9
    src, dst = small_graph(rng, n=n, p=0.5)
    x, _, Y, W, G = random_inputs(rng, prob, n, len(src))
    a, b, c = cotangents(rng, prob, n, len(src))
    dx, dY, dW = tp_backward(prob, x, Y, W, G, src, dst, n)
    ta, tb, tc = np.vdot(a, dx), np.vdot(b, dY), np.vdot(c, dW)
    gx, gY, gW, gG = tp_double_backward(prob, x, Y, W, G, a, b, c, src, dst, n)
    # L2 is linear in G; <a,dx> has no x in it, <b,dY> no Y, <c,dW> no W
    assert np.vdot(gG, G) == pytest.approx(ta + tb + tc, rel=1e-12)
    assert np.vdot(gx, x) == pytest.approx(tb + tc, rel=1e-12)
    assert np.vdot(gY, Y) == pytest.approx(ta + tc, rel=1e-12)
    assert np.vdot(gW, W) == pytest.approx(ta + tb, rel=1e-12)


@pytest.mark.parametrize("case", CASES)
def test_one_cotangent_reduces_to_forward_and_backward(case):
    rng = np.random.default_rng(23)
    prob = TPProblem.build(*case)
    n = 8
    src, dst = small_graph(rng, n=n, p=0.5)
    E = len(src)
    x, _, Y, W, G = random_inputs(rng, prob, n, E)
    a, b, c = cotangents(rng, prob, n, E)
    tol = dict(rtol=1e-12, atol=1e-12)

    # only a = d L / d(dx): dx(a...) depends on (Y, W, G)
    gx, gY, gW, gG = tp_double_backward(prob, x, Y, W, G, a, None, None, src, dst, n)
    _, dY_a, dW_a = tp_backward(prob, a, Y, W, G, src, dst, n)
    np.testing.assert_allclose(gG, tp_forward(prob, a, Y, W, src, dst, n), **tol)
    np.testing.assert_allclose(gY, dY_a, **tol)
    np.testing.assert_allclose(gW, dW_a, **tol)
    assert np.all(gx == 0.0)

    # only b = d L / d(dY)
    gx, gY, gW, gG = tp_double_backward(prob, x, Y, W, G, None, b, None, src, dst, n)
    dx_b, _, dW_b = tp_backward(prob, x, b, W, G, src, dst, n)
    np.testing.assert_allclose(gG, tp_forward(prob, x, b, W, src, dst, n), **tol)
    np.testing.assert_allclose(gx, dx_b, **tol)
    np.testing.assert_allclose(gW, dW_b, **tol)
    assert np.all(gY == 0.0)

    # only c = d L / d(dW)
    gx, gY, gW, gG = tp_double_backward(prob, x, Y, W, G, None, None, c, src, dst, n)
    dx_c, dY_c, _ = tp_backward(prob, x, Y, c, G, src, dst, n)
    np.testing.assert_allclose(gG, tp_forward(prob, x, Y, c, src, dst, n), **tol)
    np.testing.assert_allclose(gx, dx_c, **tol)
    np.testing.assert_allclose(gY, dY_c, **tol)
    assert np.all(gW == 0.0)

    # and the full result is the sum of the three (linear in the cotangents)
    full = tp_double_backward(prob, x, Y, W, G, a, b, c, src, dst, n)
    parts = [tp_double_backward(prob, x, Y, W, G, *(v if k == i else None for k, v in enumerate((a, b, c))),
                                src, dst, n) for i in range(3)]
    for t in range(4):
        np.testing.assert_allclose(full[t], parts[0][t] + parts[1][t] + parts[2][t], **tol)


@pytest.mark.parametrize("case", CASES[1:3])
def test_rotation_equivariance(case):
    rng = np.random.default_rng(24)
    prob = TPProblem.build(*case)
    n = 8
    src, dst = small_graph(rng, n=n)
    E = len(src)
    x, vec, Y, W, G = random_inputs(rng, prob, n, E)
    a, _, c = cotangents(rng, prob, n, E)
    bvec = rng.standard_normal((E, 3))
    b = sh_real(prob.sh_lmax, bvec) * rng.standard_normal((E, 1))   # transforms like Y
    q, r = np.linalg.qr(rng.standard_normal((3, 3)))
    R = q * np.sign(np.diag(r))
    if np.linalg.det(R) < 0:
        R[:, 0] *= -1
    L = max([s.l for s in prob.irreps_in] + [s.l for s in prob.irreps_out] + [prob.sh_lmax])
    Ds = {l: fitted_D(l, R, rng) for l in range(L + 1)}

    def rotY(T):
        out = T.copy()
        for l in range(prob.sh_lmax + 1):
            out[:, l * l:(l + 1) ** 2] = T[:, l * l:(l + 1) ** 2] @ Ds[l].T
        return out

    gx, gY, gW, gG = tp_double_backward(prob, x, Y, W, G, a, b, c, src, dst, n)
    r = tp_double_backward(prob, apply_D(prob.irreps_in, x, Ds), rotY(Y), W, apply_D(prob.irreps_out, G, Ds),
                           apply_D(prob.irreps_in, a, Ds), rotY(b), c, src, dst, n)
    np.testing.assert_allclose(r[0], apply_D(prob.irreps_in, gx, Ds), atol=1e-11)
    np.testing.assert_allclose(r[1], rotY(gY), atol=1e-11)
    np.testing.assert_allclose(r[2], gW, atol=1e-11)
    np.testing.assert_allclose(r[3], apply_D(prob.irreps_out, gG, Ds), atol=1e-11)


def test_no_cotangents_give_zeros_and_empty_graph():
    rng = np.random.default_rng(25)
    prob = TPProblem.build(*CASES[0])
    n = 6
    src, dst = small_graph(rng, n=n)
    x, _, Y, W, G = random_inputs(rng, prob, n, len(src))
    for t in tp_double_backward(prob, x, Y, W, G, None, None, None, src, dst, n):
        assert np.all(t == 0.0)
    e = np.zeros(0, dtype=np.int64)
    gx, gY, gW, gG = tp_double_backward(prob, x, np.zeros((0, prob.dim_sh)), np.zeros((0, prob.weight_numel)), G,
                                        x, np.zeros((0, prob.dim_sh)), np.zeros((0, prob.weight_numel)), e, e, n)
    assert gx.shape == (n, prob.dim_in) and np.all(gx == 0.0)
    assert gG.shape == (n, prob.dim_out) and np.all(gG == 0.0)
    assert gY.shape == (0, prob.dim_sh) and gW.shape == (0, prob.weight_numel)
