"""Pins for the oracle's SO(2) convolution (CPU only).

Each function of oracle/so2.py is checked against something it does not use
itself:
  * the frame rotation: orthogonality, determinant, R r_hat = z_hat;
  * the sphere quadrature: closed-form moments of x^a y^b z^c;
  * the Wigner matrices: the defining identity D Y(v) = Y(R v) at points
    outside the quadrature, the l = 1 closed form (a permutation of R), the
    least-squares fit of the tensor-product tests, D(R1 R2) = D(R1) D(R2);
  * the convolution: rotation equivariance, independence of the roll about
    the edge axis, a loop-by-loop evaluation of the definition, and -- the
    strongest pin -- equality with the (separately pinned) tensor-product
    oracle when A_m, B_m are built from the real CG coefficients at m2 = 0,
    which is what a tensor product with Y(r_hat) becomes in the edge frame;
  * the backward: the operator is linear in x and in the weights, so
    <G, f(dx)> = <grad_x, dx> and <G, f(x; dw)> = <grad_w, dw> exactly;
  * the double backward: central differences of <ggx, grad_x> + <ggw, grad_w>
    through the pinned backward (exact: linear in each input separately),
    the Euler identity in G, and the split by cotangent;
  * the gradient through the frames: central differences in D (exact: the
    energy is quadratic in D), of <grad_D, D(vec)> in the edge vectors, and
    of the whole energy in the edge vectors, plus radial invariance.
"""

from math import gamma

import numpy as np
import pytest

from oracle import TPProblem, cg_real, sh_real, tp_forward
from oracle.so2 import (edge_rotation, edge_wigner, pack_D, so2_backward, so2_forward, so2_weight_grad_entries,
                        sphere_quadrature,
                        unpack_D, weight_blocks, weight_numel, wigner_D)

from test_oracle_tp import fitted_D


def random_rotation(rng):
    q, r = np.linalg.qr(rng.standard_normal((3, 3)))
    q = q * np.sign(np.diag(r))
    if np.linalg.det(q) < 0:
        q[:, 0] *= -1
    return q


def rot_z(g):
    c, s = np.cos(g), np.sin(g)
    return np.array([[c, -s, 0.0], [s, c, 0.0], [0.0, 0.0, 1.0]])


def test_edge_rotation():
    rng = np.random.default_rng(80)
    v = rng.standard_normal((50, 3)) * rng.uniform(0.1, 5.0, (50, 1))
    v = np.concatenate([v, [[0, 0, 2.0], [0, 0, -3.0], [0, 0, 0], [1e-3, 0, -1.0], [0, 1e-9, -1.0]]])
    R = edge_rotation(v)
    for e in range(len(v)):
        np.testing.assert_allclose(R[e] @ R[e].T, np.eye(3), atol=1e-13)
        assert np.linalg.det(R[e]) == pytest.approx(1.0, abs=1e-13)
        r = np.linalg.norm(v[e])
        if r > 0:
            np.testing.assert_allclose(R[e] @ (v[e] / r), [0, 0, 1.0], atol=1e-12)
    np.testing.assert_array_equal(R[-3], np.eye(3))
    np.testing.assert_array_equal(R[-4], np.diag([1.0, -1.0, -1.0]))


@pytest.mark.parametrize("degree", [0, 2, 6, 8])
def test_quadrature_moments(degree):
    pts, w = sphere_quadrature(degree)
    assert w.sum() == pytest.approx(4 * np.pi, rel=1e-14)
    for a in range(degree + 1):
        for b in range(degree + 1 - a):
            for c in range(degree + 1 - a - b):
                q = np.sum(w * pts[:, 0] ** a * pts[:, 1] ** b * pts[:, 2] ** c)
                if a % 2 or b % 2 or c % 2:
                    exact = 0.0
                else:   # integral of x^a y^b z^c over the unit sphere
                    exact = 2 * gamma((a + 1) / 2) * gamma((b + 1) / 2) * gamma((c + 1) / 2) / gamma((a + b + c + 3) / 2)
                assert q == pytest.approx(exact, abs=1e-13), (a, b, c)


@pytest.mark.parametrize("lmax", [1, 3, 4])
def test_wigner_defining_identity(lmax):
    rng = np.random.default_rng(81 + lmax)
    Rs = np.stack([random_rotation(rng) for _ in range(6)])
    Ds = wigner_D(lmax, Rs)
    v = rng.standard_normal((30, 3))
    for e in range(len(Rs)):
        for l in range(lmax + 1):
            sl = slice(l * l, (l + 1) ** 2)
            np.testing.assert_allclose(sh_real(lmax, v @ Rs[e].T)[:, sl], sh_real(lmax, v)[:, sl] @ Ds[l][e].T,
                                       atol=1e-12)
            np.testing.assert_allclose(Ds[l][e] @ Ds[l][e].T, np.eye(2 * l + 1), atol=1e-12)
            np.testing.assert_allclose(Ds[l][e], fitted_D(l, Rs[e], rng), atol=1e-11)


def test_wigner_l1_closed_form_and_homomorphism():
    rng = np.random.default_rng(85)
    R1, R2 = random_rotation(rng), random_rotation(rng)
    P = np.zeros((3, 3))
    P[0, 1] = P[1, 2] = P[2, 0] = 1.0            # Y_1 = sqrt(3) (y, z, x)
    D1 = wigner_D(1, R1[None])[1][0]
    np.testing.assert_allclose(D1, P @ R1 @ P.T, atol=1e-13)
    a, b, ab = wigner_D(4, np.stack([R1, R2, R1 @ R2]))[4]
    np.testing.assert_allclose(ab, a @ b, atol=1e-12)


def test_edge_frame_aligns_harmonics():
    rng = np.random.default_rng(86)
    v = rng.standard_normal((40, 3))
    Dl = unpack_D(edge_wigner(3, v), 3)
    Y = sh_real(3, v)
    for l in range(4):
        rot = np.einsum("emn,en->em", Dl[l], Y[:, l * l:(l + 1) ** 2])
        want = np.zeros_like(rot)
        want[:, l] = np.sqrt(2 * l + 1)           # Y_l(z_hat): only m = 0
        np.testing.assert_allclose(rot, want, atol=1e-12)


def make_graph(rng, n, E):
    src = rng.integers(0, n, E)
    dst = rng.integers(0, n, E)
    vec = rng.standard_normal((E, 3)) * rng.uniform(0.5, 4.0, (E, 1))
    return src, dst, vec


def rotate_feats(x, lmax, C, Ds):
    out = x.copy()
    for l in range(lmax + 1):
        sl = slice(C * l * l, C * (l + 1) ** 2)
        out[:, sl] = (x[:, sl].reshape(len(x), C, 2 * l + 1) @ Ds[l].T).reshape(len(x), -1)
    return out


@pytest.mark.parametrize("lmax,C", [(1, 3), (2, 2), (3, 2)])
def test_equivariance(lmax, C):
    rng = np.random.default_rng(90 + lmax)
    n, E = 7, 40
    src, dst, vec = make_graph(rng, n, E)
    x = rng.standard_normal((n, C * (lmax + 1) ** 2))
    w = rng.standard_normal(weight_numel(lmax, C))
    out = so2_forward(lmax, C, x, edge_wigner(lmax, vec), w, src, dst, n)
    Q = random_rotation(rng)
    DQ = [d[0] for d in wigner_D(lmax, Q[None])]
    out_r = so2_forward(lmax, C, rotate_feats(x, lmax, C, DQ), edge_wigner(lmax, vec @ Q.T), w, src, dst, n)
    np.testing.assert_allclose(out_r, rotate_feats(out, lmax, C, DQ), atol=1e-11)


def test_roll_invariance():
    rng = np.random.default_rng(95)
    lmax, C, n, E = 3, 3, 6, 30
    src, dst, vec = make_graph(rng, n, E)
    x = rng.standard_normal((n, C * 16))
    w = rng.standard_normal(weight_numel(lmax, C))
    R = edge_rotation(vec)
    rolled = np.stack([rot_z(g) @ R[e] for e, g in enumerate(rng.uniform(0, 2 * np.pi, E))])
    a = so2_forward(lmax, C, x, pack_D(wigner_D(lmax, R)), w, src, dst, n)
    b = so2_forward(lmax, C, x, pack_D(wigner_D(lmax, rolled)), w, src, dst, n)
    np.testing.assert_allclose(a, b, atol=1e-11)


def brute_forward(lmax, C, x, D, w, src, dst, n):
    """The definition, one scalar at a time."""
    Dl = unpack_D(D, lmax)
    blocks = {b[0] + str(b[1]): (b[2], b[3]) for b in weight_blocks(lmax, C)}

    def Wm(name, m, o, i):
        off, K = blocks[name + str(m)]
        return w[off + o * K + i]

    out = np.zeros((n, C * (lmax + 1) ** 2))
    for e in range(len(src)):
        xt = {}
        for l in range(lmax + 1):
            for c in range(C):
                for mi in range(-l, l + 1):
                    xt[l, c, mi] = sum(Dl[l][e, mi + l, ni + l] * x[src[e], C * l * l + c * (2 * l + 1) + ni + l]
                                       for ni in range(-l, l + 1))
        yt = {}
        for l3 in range(lmax + 1):
            for c3 in range(C):
                for m3 in range(-l3, l3 + 1):
                    m = abs(m3)
                    o = (l3 - m) * C + c3
                    s = 0.0
                    for l1 in range(m, lmax + 1):
                        for c1 in range(C):
                            i = (l1 - m) * C + c1
                            if m == 0:
                                s += Wm("A", 0, o, i) * xt[l1, c1, 0]
                            elif m3 > 0:
                                s += Wm("A", m, o, i) * xt[l1, c1, m] - Wm("B", m, o, i) * xt[l1, c1, -m]
                            else:
                                s += Wm("B", m, o, i) * xt[l1, c1, m] + Wm("A", m, o, i) * xt[l1, c1, -m]
                    yt[l3, c3, m3] = s
        for l in range(lmax + 1):
            for c in range(C):
                for ni in range(-l, l + 1):
                    out[dst[e], C * l * l + c * (2 * l + 1) + ni + l] += sum(
                        Dl[l][e, mi + l, ni + l] * yt[l, c, mi] for mi in range(-l, l + 1))
    return out


def test_matches_brute_force():
    rng = np.random.default_rng(96)
    lmax, C, n, E = 2, 2, 5, 12
    src, dst, vec = make_graph(rng, n, E)
    x = rng.standard_normal((n, C * 9))
    w = rng.standard_normal(weight_numel(lmax, C))
    D = edge_wigner(lmax, vec)
    np.testing.assert_allclose(so2_forward(lmax, C, x, D, w, src, dst, n), brute_forward(lmax, C, x, D, w, src, dst, n),
                               atol=1e-12)


def escn_weights(prob, lmax, C, w_path):
    """A_m, B_m of the tensor product with Y(r_hat) seen in the edge frame:
    Y_l2(z_hat) = sqrt(2 l2 + 1) at m2 = 0 only, so path p = (l1, l2, l3)
    maps x~[l1][u][m1] to y~[l3][u][m3] with coefficient
    w[p,u] sqrt(2 l2 + 1) C_p[m1, 0, m3], nonzero only for |m1| = |m3|."""
    W = np.zeros(weight_numel(lmax, C))
    blocks = {b[0] + str(b[1]): (b[2], b[3]) for b in weight_blocks(lmax, C)}
    for p, (s1, l2, s3) in enumerate(prob.paths):
        l1, l3 = prob.irreps_in[s1].l, prob.irreps_out[s3].l
        cg = cg_real(l1, l2, l3)[:, l2, :] * np.sqrt(2 * l2 + 1)      # [m1 + l1, m3 + l3]
        for m1 in range(-l1, l1 + 1):
            for m3 in range(-l3, l3 + 1):
                if abs(m1) != abs(m3):
                    assert cg[m1 + l1, m3 + l3] == 0.0
        for m in range(0, min(l1, l3) + 1):
            a = cg[l1 + m, l3 + m]
            if m > 0:
                b = cg[l1 + m, l3 - m]
                # the complex-multiplication form the SO(2) map assumes
                assert cg[l1 - m, l3 - m] == pytest.approx(a, abs=1e-14)
                assert cg[l1 - m, l3 + m] == pytest.approx(-b, abs=1e-14)
            for u in range(C):
                o, i = (l3 - m) * C + u, (l1 - m) * C + u
                offA, K = blocks["A" + str(m)]
                W[offA + o * K + i] += w_path[p, u] * a
                if m > 0:
                    offB, _ = blocks["B" + str(m)]
                    W[offB + o * K + i] += w_path[p, u] * b
    return W


@pytest.mark.parametrize("case", [("3x0e+3x1o+3x2e", 2, "3x0e+3x1o+3x2e"),
                                  ("2x0e+2x1o+2x2e+2x3o", 3, "2x0e+2x1o+2x2e+2x3o"),
                                  ("2x0e+2x1o+2x2e", 2, "2x0o+2x1e+2x2o"),        # odd paths: B_m only
                                  ("2x0e+2x1e+2x2e+2x3e", 3, "2x0e+2x1e+2x2e+2x3e")])  # both parities
def test_equals_tensor_product_in_edge_frame(case):
    rng = np.random.default_rng(97)
    prob = TPProblem.build(*case)
    lmax, C = prob.sh_lmax, prob.irreps_in[0].mul
    n, E = 8, 50
    src, dst, vec = make_graph(rng, n, E)
    x = rng.standard_normal((n, prob.dim_in))
    w_path = rng.standard_normal((len(prob.paths), C))
    W_edges = np.concatenate([np.tile(w_path[p], (E, 1)) for p in range(len(prob.paths))], axis=1)
    ref = tp_forward(prob, x, sh_real(lmax, vec), W_edges, src, dst, n)
    got = so2_forward(lmax, C, x, edge_wigner(lmax, vec), escn_weights(prob, lmax, C, w_path), src, dst, n)
    np.testing.assert_allclose(got, ref, atol=1e-11 * np.abs(ref).max())


@pytest.mark.parametrize("lmax,C", [(1, 2), (3, 3)])
def test_backward_by_linearity(lmax, C):
    rng = np.random.default_rng(98 + lmax)
    n, E = 9, 60
    src, dst, vec = make_graph(rng, n, E)
    D = edge_wigner(lmax, vec)
    d = C * (lmax + 1) ** 2
    x = rng.standard_normal((n, d))
    w = rng.standard_normal(weight_numel(lmax, C))
    G = rng.standard_normal((n, d))
    gx, gw = so2_backward(lmax, C, x, D, w, G, src, dst, n)
    for _ in range(3):
        dx = rng.standard_normal((n, d))
        dw = rng.standard_normal(len(w))
        lhs_x = np.vdot(G, so2_forward(lmax, C, dx, D, w, src, dst, n))
        lhs_w = np.vdot(G, so2_forward(lmax, C, x, D, dw, src, dst, n))
        assert np.vdot(gx, dx) == pytest.approx(lhs_x, rel=1e-11)
        assert np.vdot(gw, dw) == pytest.approx(lhs_w, rel=1e-11)
    # every weight block is reached
    for _, _, off, K in weight_blocks(lmax, C):
        assert np.abs(gw[off:off + K * K]).max() > 0


@pytest.mark.parametrize("lmax,C", [(1, 2), (2, 2), (3, 1)])
def test_weight_grad_entries_by_one_hot_weights(lmax, C):
    """Each map-gradient entry, evaluated on its own, equals <G, f(x; e_j)>:
    the forward with a one-hot weight vector (the operator is linear in the
    weights), for every entry of every block."""
    rng = np.random.default_rng(97 + lmax)
    n, E = 8, 50
    src, dst, vec = make_graph(rng, n, E)
    D = edge_wigner(lmax, vec)
    d = C * (lmax + 1) ** 2
    x, G = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    nw = weight_numel(lmax, C)
    got = so2_weight_grad_entries(lmax, C, x, D, G, src, dst, np.arange(nw))
    want = np.empty(nw)
    for j in range(nw):
        e = np.zeros(nw)
        e[j] = 1.0
        want[j] = np.vdot(G, so2_forward(lmax, C, x, D, e, src, dst, n))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12 * np.abs(want).max())
    # and the whole backward agrees with it
    _, gw = so2_backward(lmax, C, x, D, rng.standard_normal(nw), G, src, dst, n)
    np.testing.assert_allclose(gw, want, rtol=0, atol=1e-12 * np.abs(want).max())


def test_isolated_nodes_and_no_edges():
    rng = np.random.default_rng(99)
    lmax, C, n = 2, 2, 4
    w = rng.standard_normal(weight_numel(lmax, C))
    x = rng.standard_normal((n, C * 9))
    e = np.zeros(0, np.int64)
    out = so2_forward(lmax, C, x, np.zeros((0, 35)), w, e, e, n)
    assert out.shape == (n, 18) and np.all(out == 0)
    gx, gw = so2_backward(lmax, C, x, np.zeros((0, 35)), w, x, e, e, n)
    assert np.all(gx == 0) and np.all(gw == 0)


@pytest.mark.parametrize("lmax,C", [(1, 2), (2, 2), (3, 2)])
def test_double_backward_by_differences(lmax, C):
    """L2 = <ggx, grad_x> + <ggw, grad_w> is linear in each of x, w, G
    separately, so a central difference along any direction is exact up to
    rounding: it pins every output of so2_double_backward against the
    (separately pinned) backward."""
    from oracle.so2 import so2_double_backward
    rng = np.random.default_rng(110 + lmax)
    n, E = 7, 45
    src, dst, vec = make_graph(rng, n, E)
    D = edge_wigner(lmax, vec)
    d, nw = C * (lmax + 1) ** 2, weight_numel(lmax, C)
    x, G = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    w = rng.standard_normal(nw)
    ggx, ggw = rng.standard_normal((n, d)), rng.standard_normal(nw)

    def L2(x_, w_, G_):
        gx, gw = so2_backward(lmax, C, x_, D, w_, G_, src, dst, n)
        return np.vdot(ggx, gx) + np.vdot(ggw, gw)

    gx2, gw2, gG2 = so2_double_backward(lmax, C, x, D, w, G, ggx, ggw, src, dst, n)
    h = 0.5
    for _ in range(2):
        dx, dw, dG = rng.standard_normal((n, d)), rng.standard_normal(nw), rng.standard_normal((n, d))
        fx = (L2(x + h * dx, w, G) - L2(x - h * dx, w, G)) / (2 * h)
        fw = (L2(x, w + h * dw, G) - L2(x, w - h * dw, G)) / (2 * h)
        fG = (L2(x, w, G + h * dG) - L2(x, w, G - h * dG)) / (2 * h)
        assert np.vdot(gx2, dx) == pytest.approx(fx, rel=1e-10, abs=1e-9)
        assert np.vdot(gw2, dw) == pytest.approx(fw, rel=1e-10, abs=1e-9)
        assert np.vdot(gG2, dG) == pytest.approx(fG, rel=1e-10, abs=1e-9)
    # Euler identity: L2 is homogeneous of degree 1 in G
    assert np.vdot(gG2, G) == pytest.approx(L2(x, w, G), rel=1e-10)
    # one cotangent at a time
    gx_a, gw_a, gG_a = so2_double_backward(lmax, C, x, D, w, G, ggx, None, src, dst, n)
    assert np.all(gx_a == 0) and np.abs(gw_a).max() > 0
    gx_b, gw_b, gG_b = so2_double_backward(lmax, C, x, D, w, G, None, ggw, src, dst, n)
    assert np.all(gw_b == 0) and np.abs(gx_b).max() > 0
    np.testing.assert_allclose(gG_a + gG_b, gG2, atol=1e-12)


def test_frames_backward_exact_in_D():
    """<G, out> is quadratic in the Wigner blocks (they enter twice), so a
    central difference in D is exact up to rounding."""
    from oracle.so2 import so2_frames_backward
    rng = np.random.default_rng(120)
    lmax, C, n, E = 2, 2, 6, 25
    src, dst, vec = make_graph(rng, n, E)
    D = edge_wigner(lmax, vec)
    x, G = rng.standard_normal((n, C * 9)), rng.standard_normal((n, C * 9))
    w = rng.standard_normal(weight_numel(lmax, C))
    gD = so2_frames_backward(lmax, C, x, D, w, G, src, dst, n)
    f = lambda D_: np.vdot(G, so2_forward(lmax, C, x, D_, w, src, dst, n))  # noqa: E731
    for _ in range(3):
        dD = rng.standard_normal(D.shape)
        fd = (f(D + 0.5 * dD) - f(D - 0.5 * dD)) / 1.0
        assert np.vdot(gD, dD) == pytest.approx(fd, rel=1e-10)


@pytest.mark.parametrize("lmax", [1, 3])
def test_rotations_backward_by_differences(lmax):
    from oracle.so2 import rotations_backward
    rng = np.random.default_rng(121 + lmax)
    vec = rng.standard_normal((12, 3)) * 2.0
    gD = rng.standard_normal(edge_wigner(lmax, vec).shape)
    g = rotations_backward(lmax, vec, gD)
    h = 1e-6
    for j in range(3):
        dv = np.zeros_like(vec)
        dv[:, j] = h
        fd = (np.sum(gD * edge_wigner(lmax, vec + dv), axis=1) - np.sum(gD * edge_wigner(lmax, vec - dv), axis=1)) / (2 * h)
        np.testing.assert_allclose(g[:, j], fd, rtol=1e-6, atol=1e-7)


def test_force_through_the_frames():
    """The whole chain: d<G, out>/dvec from so2_frames_backward and
    rotations_backward against central differences of the energy in the edge
    vectors (the energy does not depend on the frames' roll, so this also
    checks the chain against the frame convention)."""
    from oracle.so2 import rotations_backward, so2_frames_backward
    rng = np.random.default_rng(125)
    lmax, C, n, E = 3, 2, 6, 20
    src, dst, vec = make_graph(rng, n, E)
    x, G = rng.standard_normal((n, C * 16)), rng.standard_normal((n, C * 16))
    w = rng.standard_normal(weight_numel(lmax, C))
    gvec = rotations_backward(lmax, vec, so2_frames_backward(lmax, C, x, edge_wigner(lmax, vec), w, G, src, dst, n))
    energy = lambda v: np.vdot(G, so2_forward(lmax, C, x, edge_wigner(lmax, v), w, src, dst, n))  # noqa: E731
    h = 1e-6
    for _ in range(3):
        dv = rng.standard_normal(vec.shape)
        fd = (energy(vec + h * dv) - energy(vec - h * dv)) / (2 * h)
        assert np.vdot(gvec, dv) == pytest.approx(fd, rel=1e-6, abs=1e-8)
    # radial invariance: the frames depend on the direction only
    np.testing.assert_allclose(np.einsum("ej,ej->e", gvec, vec), 0.0, atol=1e-9)


@pytest.mark.parametrize("lmax", [1, 3])
def test_rotations_jvp_by_differences_and_adjoint(lmax):
    """The frames' directional derivative against central differences of
    edge_wigner, and its adjoint relation with rotations_backward (pinned by
    differences above): <jvp(dv), gD> = <dv, backward(gD)> per edge."""
    from oracle.so2 import rotations_backward, rotations_jvp
    rng = np.random.default_rng(130 + lmax)
    vec = rng.standard_normal((10, 3)) * 2.0
    vec[3] = [0.0, 0.0, 1.5]                         # on the z axis: convention, zero
    dv = rng.standard_normal(vec.shape)
    jv = rotations_jvp(lmax, vec, dv)
    h = 1e-6
    fd = (edge_wigner(lmax, vec + h * dv) - edge_wigner(lmax, vec - h * dv)) / (2 * h)
    keep = np.arange(len(vec)) != 3
    np.testing.assert_allclose(jv[keep], fd[keep], rtol=1e-6, atol=1e-7)
    assert np.all(jv[3] == 0)
    gD = rng.standard_normal(jv.shape)
    np.testing.assert_allclose(np.sum(jv * gD, axis=1), np.sum(dv * rotations_backward(lmax, vec, gD), axis=1),
                               rtol=1e-10, atol=1e-12)
    # radial invariance: moving the vector along itself does not change the frame
    np.testing.assert_allclose(rotations_jvp(lmax, vec, vec), 0.0, atol=1e-12)


@pytest.mark.parametrize("lmax,C", [(1, 2), (3, 2)])
def test_frames_double_backward_by_linearity(lmax, C):
    """S = <dD, so2_frames_backward(x, w, G)> is linear in x, in the weights
    and in G separately, so S(v + u) - S(v) = <grad_v, u> exactly (up to
    rounding) for each of them, against the pinned so2_frames_backward."""
    from oracle.so2 import so2_frames_backward, so2_frames_double_backward
    rng = np.random.default_rng(140 + lmax)
    n, E = 7, 30
    src, dst, vec = make_graph(rng, n, E)
    d = C * (lmax + 1) ** 2
    D = edge_wigner(lmax, vec)
    x, G = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    w = rng.standard_normal(weight_numel(lmax, C))
    dD = rng.standard_normal(D.shape)
    gx, gw, gG = so2_frames_double_backward(lmax, C, x, D, w, G, dD, src, dst, n)
    S = lambda x_, w_, G_: np.vdot(dD, so2_frames_backward(lmax, C, x_, D, w_, G_, src, dst, n))  # noqa: E731
    s0 = S(x, w, G)
    for _ in range(2):
        ux, uw, uG = rng.standard_normal(x.shape), rng.standard_normal(w.shape), rng.standard_normal(G.shape)
        assert S(x + ux, w, G) - s0 == pytest.approx(np.vdot(gx, ux), rel=1e-9, abs=1e-9)
        assert S(x, w + uw, G) - s0 == pytest.approx(np.vdot(gw, uw), rel=1e-9, abs=1e-9)
        assert S(x, w, G + uG) - s0 == pytest.approx(np.vdot(gG, uG), rel=1e-9, abs=1e-9)
    # with dD = D the mixed terms are the two halves of the first derivative
    # in D taken along itself: S = 2 <G, out>, so grad_G = 2 out
    _, _, gG2 = so2_frames_double_backward(lmax, C, x, D, w, G, D, src, dst, n)
    np.testing.assert_allclose(gG2, 2.0 * so2_forward(lmax, C, x, D, w, src, dst, n), rtol=1e-10, atol=1e-10)
    # the two terms of each gradient swap when D and dD swap, and the grad_G
    # terms sum to the polarisation of the (quadratic in D) forward
    p1 = so2_frames_double_backward(lmax, C, x, D, w, G, dD, src, dst, n, parts=True)
    p2 = so2_frames_double_backward(lmax, C, x, dD, w, G, D, src, dst, n, parts=True)
    for (a1, b1), (a2, b2), full in zip(p1, p2, (gx, gw, gG)):
        np.testing.assert_allclose(a1, b2, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(b1, a2, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(a1 + b1, full, rtol=1e-12, atol=1e-12)
    fwd = lambda D_: so2_forward(lmax, C, x, D_, w, src, dst, n)  # noqa: E731
    np.testing.assert_allclose(fwd(D + dD) - fwd(D - dD), 2.0 * (p1[2][0] + p1[2][1]), rtol=1e-10, atol=1e-10)


def roll_generator(l):
    """Generator of rotations about the edge axis on the real degree-l
    harmonics: the (m, -m) pair turns at rate m."""
    J = np.zeros((2 * l + 1, 2 * l + 1))
    for m in range(1, l + 1):
        J[l - m, l + m] = m
        J[l + m, l - m] = -m
    return J


@pytest.mark.parametrize("lmax,C", [(1, 2), (3, 2)])
def test_roll_direction_is_invisible_to_the_frame_gradients(lmax, C):
    """Rolling a frame about its edge axis leaves the convolution unchanged
    (test_roll_invariance), so with J the roll generator (checked against the
    Wigner blocks of small rolls): grad_D of each edge is orthogonal to J D_e,
    and the mixed second derivatives do not change when dD_e moves along
    J D_e, whatever dD is."""
    from oracle.so2 import so2_frames_backward, so2_frames_double_backward
    rng = np.random.default_rng(150 + lmax)
    h = 1e-6
    Dp, Dm = wigner_D(lmax, rot_z(h)[None]), wigner_D(lmax, rot_z(-h)[None])
    for l in range(lmax + 1):
        np.testing.assert_allclose((Dp[l][0] - Dm[l][0]) / (2 * h), roll_generator(l), atol=1e-8)
    n, E = 7, 30
    src, dst, vec = make_graph(rng, n, E)
    d = C * (lmax + 1) ** 2
    D = edge_wigner(lmax, vec)
    x, G = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    w = rng.standard_normal(weight_numel(lmax, C))
    JD = pack_D([roll_generator(l)[None] @ b for l, b in enumerate(unpack_D(D, lmax))])
    gD = so2_frames_backward(lmax, C, x, D, w, G, src, dst, n)
    assert np.max(np.abs(np.sum(gD * JD, axis=1))) <= 1e-11 * np.max(np.abs(gD)) * np.max(np.abs(JD)) * D.shape[1]
    dD = rng.standard_normal(D.shape)
    c = rng.standard_normal((E, 1)) * 50.0
    a = so2_frames_double_backward(lmax, C, x, D, w, G, dD, src, dst, n)
    b = so2_frames_double_backward(lmax, C, x, D, w, G, dD + c * JD, src, dst, n)
    for u, v in zip(a, b):
        np.testing.assert_allclose(u, v, rtol=0, atol=1e-10 * np.max(np.abs(u)) * 50)
