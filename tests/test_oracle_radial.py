"""Pins for the oracle's radial-weights step (CPU only).

radial_forward is the convolution with W = h M; radial_backward gives the
gradients of <G, out> with respect to x, Y, h and M.  Pinned against the
already pinned convolution oracle and the mathematics, never its own formulas:

* the output is linear in each of x, Y, h and M separately, so a central
  difference of <G, out> along any direction equals the gradient's inner
  product with that direction, exactly up to rounding;
* one-hot hidden features select rows of M: the output equals the
  convolution with those rows as weights (which fixes M's orientation);
* M = I (H = P U): h is W itself, dh is the convolution's dW and dM = h^T dW
  sums dW over edges weighted by W.
"""

import numpy as np
import pytest

from oracle import TPProblem, radial_backward, radial_forward, tp_backward, tp_forward

from test_oracle_tp import CASES, random_inputs, small_graph


def setup(case, seed, H=5):
    rng = np.random.default_rng(seed)
    prob = TPProblem.build(*case)
    src, dst = small_graph(rng)
    n = 7
    x, _, Y, _, G = random_inputs(rng, prob, n, len(src))
    h = rng.standard_normal((len(src), H))
    M = rng.standard_normal((H, prob.weight_numel))
    return rng, prob, src, dst, n, x, Y, h, M, G


@pytest.mark.parametrize("case", CASES)
def test_differences_are_exact(case):
    rng, prob, src, dst, n, x, Y, h, M, G = setup(case, 61)
    dx, dY, dh, dM = radial_backward(prob, x, Y, h, M, G, src, dst, n)
    E = lambda x_, Y_, h_, M_: np.vdot(G, radial_forward(prob, x_, Y_, h_, M_, src, dst, n))  # noqa: E731
    for _ in range(2):
        ux, uY = rng.standard_normal(x.shape), rng.standard_normal(Y.shape)
        uh, uM = rng.standard_normal(h.shape), rng.standard_normal(M.shape)
        for s in (1.0, 1e-3):
            assert (E(x + s * ux, Y, h, M) - E(x - s * ux, Y, h, M)) / (2 * s) == pytest.approx(np.vdot(dx, ux), rel=1e-9, abs=1e-9)
            assert (E(x, Y + s * uY, h, M) - E(x, Y - s * uY, h, M)) / (2 * s) == pytest.approx(np.vdot(dY, uY), rel=1e-9, abs=1e-9)
            assert (E(x, Y, h + s * uh, M) - E(x, Y, h - s * uh, M)) / (2 * s) == pytest.approx(np.vdot(dh, uh), rel=1e-9, abs=1e-9)
            assert (E(x, Y, h, M + s * uM) - E(x, Y, h, M - s * uM)) / (2 * s) == pytest.approx(np.vdot(dM, uM), rel=1e-9, abs=1e-9)


def test_one_hot_features_select_rows():
    rng, prob, src, dst, n, x, Y, h, M, G = setup(CASES[1], 62, H=4)
    k = rng.integers(0, 4, len(src))
    onehot = np.eye(4)[k]
    np.testing.assert_allclose(radial_forward(prob, x, Y, onehot, M, src, dst, n),
                               tp_forward(prob, x, Y, M[k], src, dst, n), rtol=1e-12, atol=1e-12)


def test_identity_layer_is_the_plain_convolution():
    rng, prob, src, dst, n, x, Y, _, _, G = setup(CASES[0], 63)
    P = prob.weight_numel
    W = rng.standard_normal((len(src), P))
    dx, dY, dh, dM = radial_backward(prob, x, Y, W, np.eye(P), G, src, dst, n)
    rx, rY, rW = tp_backward(prob, x, Y, W, G, src, dst, n)
    for a, b in ((dx, rx), (dY, rY), (dh, rW)):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dM, sum(np.outer(W[e], rW[e]) for e in range(len(src))), rtol=1e-12, atol=1e-12)
