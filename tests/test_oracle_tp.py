"""Pins for the oracle's forward and backward (CPU only).

Checks: naive nested-loop brute force, rotation and inversion equivariance with
Wigner-D matrices fitted from the harmonics themselves, the trilinear identities
<G,out> = <x,dx> = <Y,dY> = <W,dW>, finite differences, and closed-form special
cases (scalar channels = sparse matrix product, the dot-product path, edges
along z).
"""

import itertools
from math import sqrt

import numpy as np
import pytest
import scipy.sparse as sp

from oracle import TPProblem, cg_real, sh_real, tp_backward, tp_forward


def small_graph(rng, n=7, p=0.45, self_loops=False):
    src, dst = [], []
    for i, j in itertools.product(range(n), repeat=2):
        if (i != j or self_loops) and rng.random() < p:
            dst.append(i)
            src.append(j)
    # leave the last node without in-edges and another without out-edges
    keep = [k for k in range(len(src)) if dst[k] != n - 1 and src[k] != n - 2]
    return np.array(src)[keep], np.array(dst)[keep]


def random_inputs(rng, prob, n, E):
    x = rng.standard_normal((n, prob.dim_in))
    vec = rng.standard_normal((E, 3))
    Y = sh_real(prob.sh_lmax, vec)
    W = rng.standard_normal((E, prob.weight_numel))
    G = rng.standard_normal((n, prob.dim_out))
    return x, vec, Y, W, G


CASES = [
    ("2x0e+2x1o", 1, "2x0e+2x1o"),
    ("2x0e+2x1o+2x2e", 2, "2x0e+2x1o+2x2e"),
    ("3x1o+3x0e", 2, "3x1e+3x2o+3x0o"),          # odd-sum paths, unsorted segments
    ("1x0e+1x1o+1x2e+1x3o", 3, "1x0e+1x1o+1x2e+1x3o"),
]


def naive(prob, x, Y, W, G, src, dst, n):
    out = np.zeros((n, prob.dim_out))
    dx = np.zeros_like(x)
    dY = np.zeros_like(Y)
    dW = np.zeros_like(W)
    oi, oo = prob.irreps_in.offsets(), prob.irreps_out.offsets()
    for e in range(len(src)):
        j, i = src[e], dst[e]
        for p, (s1, l2, s3) in enumerate(prob.paths):
            l1, _, l3 = prob.path_ls(p)
            C = cg_real(l1, l2, l3)
            for u in range(prob.irreps_in[s1].mul):
                w = W[e, prob.weight_offsets[p] + u]
                for m1 in range(2 * l1 + 1):
                    for m2 in range(2 * l2 + 1):
                        for m3 in range(2 * l3 + 1):
                            c = C[m1, m2, m3]
                            if c == 0.0:
                                continue
                            a = oi[s1] + u * (2 * l1 + 1) + m1
                            b = l2 * l2 + m2
                            d = oo[s3] + u * (2 * l3 + 1) + m3
                            out[i, d] += w * c * x[j, a] * Y[e, b]
                            dx[j, a] += w * c * Y[e, b] * G[i, d]
                            dY[e, b] += w * c * x[j, a] * G[i, d]
                            dW[e, prob.weight_offsets[p] + u] += c * x[j, a] * Y[e, b] * G[i, d]
    return out, dx, dY, dW


@pytest.mark.parametrize("case", CASES)
def test_brute_force(case):
    rng = np.random.default_rng(11)
    prob = TPProblem.build(*case)
    src, dst = small_graph(rng, n=6)
    x, _, Y, W, G = random_inputs(rng, prob, 6, len(src))
    ref = naive(prob, x, Y, W, G, src, dst, 6)
    out = tp_forward(prob, x, Y, W, src, dst, 6, chunk=5)
    dx, dY, dW = tp_backward(prob, x, Y, W, G, src, dst, 6, chunk=5)
    for a, b in zip((out, dx, dY, dW), ref):
        np.testing.assert_allclose(a, b, atol=1e-12)
    assert np.all(out[5] == 0.0)   # no in-edges
    assert np.all(dx[4] == 0.0)    # no out-edges


def fitted_D(l, R, rng):
    pts = rng.standard_normal((4 * l + 8, 3))
    A = sh_real(l, pts)[:, l * l:]
    B = sh_real(l, pts @ R.T)[:, l * l:]
    D = B.T @ np.linalg.pinv(A.T)
    np.testing.assert_allclose(D @ D.T, np.eye(2 * l + 1), atol=1e-12)
    return D


def apply_D(prob_irreps, feats, Ds, parity=None):
    out = feats.copy()
    for s, seg in enumerate(prob_irreps):
        sl = prob_irreps.slice(s)
        blk = feats[:, sl].reshape(len(feats), seg.mul, 2 * seg.l + 1)
        if parity is None:
            blk = blk @ Ds[seg.l].T
        else:
            blk = blk * seg.p
        out[:, sl] = blk.reshape(len(feats), -1)
    return out


@pytest.mark.parametrize("case", CASES)
def test_rotation_equivariance(case):
    rng = np.random.default_rng(12)
    prob = TPProblem.build(*case)
    n = 8
    src, dst = small_graph(rng, n=n)
    x, vec, Y, W, G = random_inputs(rng, prob, n, len(src))
    q, r = np.linalg.qr(rng.standard_normal((3, 3)))
    R = q * np.sign(np.diag(r))
    if np.linalg.det(R) < 0:
        R[:, 0] *= -1
    L = max([s.l for s in prob.irreps_in] + [s.l for s in prob.irreps_out] + [prob.sh_lmax])
    Ds = {l: fitted_D(l, R, rng) for l in range(L + 1)}
    Yr = sh_real(prob.sh_lmax, vec @ R.T)
    xr = apply_D(prob.irreps_in, x, Ds)
    Gr = apply_D(prob.irreps_out, G, Ds)
    out = tp_forward(prob, x, Y, W, src, dst, n)
    out_r = tp_forward(prob, xr, Yr, W, src, dst, n)
    np.testing.assert_allclose(out_r, apply_D(prob.irreps_out, out, Ds), atol=1e-12)
    dx, dY, dW = tp_backward(prob, x, Y, W, G, src, dst, n)
    dxr, dYr, dWr = tp_backward(prob, xr, Yr, W, Gr, src, dst, n)
    np.testing.assert_allclose(dxr, apply_D(prob.irreps_in, dx, Ds), atol=1e-12)
    for l in range(prob.sh_lmax + 1):
        np.testing.assert_allclose(dYr[:, l * l:(l + 1) ** 2], dY[:, l * l:(l + 1) ** 2] @ Ds[l].T, atol=1e-12)
    np.testing.assert_allclose(dWr, dW, atol=1e-12)


@pytest.mark.parametrize("case", CASES)
def test_inversion_parity(case):
    rng = np.random.default_rng(13)
    prob = TPProblem.build(*case)
    n = 7
    src, dst = small_graph(rng, n=n)
    x, vec, Y, W, G = random_inputs(rng, prob, n, len(src))
    Yi = sh_real(prob.sh_lmax, -vec)
    for l in range(prob.sh_lmax + 1):
        np.testing.assert_allclose(Yi[:, l * l:(l + 1) ** 2], (-1) ** l * Y[:, l * l:(l + 1) ** 2], atol=1e-13)
    xi = apply_D(prob.irreps_in, x, None, parity=True)
    out = tp_forward(prob, x, Y, W, src, dst, n)
    out_i = tp_forward(prob, xi, Yi, W, src, dst, n)
    np.testing.assert_allclose(out_i, apply_D(prob.irreps_out, out, None, parity=True), atol=1e-12)


@pytest.mark.parametrize("case", CASES)
def test_trilinear_identities_and_finite_differences(case):
    rng = np.random.default_rng(14)
    prob = TPProblem.build(*case)
    n = 9
    src, dst = small_graph(rng, n=n, p=0.5)
    x, _, Y, W, G = random_inputs(rng, prob, n, len(src))
    out = tp_forward(prob, x, Y, W, src, dst, n)
    dx, dY, dW = tp_backward(prob, x, Y, W, G, src, dst, n)
    ref = np.vdot(G, out)
    for a, b in ((x, dx), (Y, dY), (W, dW)):
        assert np.vdot(a, b) == pytest.approx(ref, rel=1e-12)
    # the map is linear in each argument, so a central difference is exact up to rounding
    h = 0.37
    for name, grad in (("x", dx), ("Y", dY), ("W", dW)):
        args = dict(x=x, Y=Y, W=W)
        d = rng.standard_normal(args[name].shape)
        plus = dict(args, **{name: args[name] + h * d})
        minus = dict(args, **{name: args[name] - h * d})
        fd = (np.vdot(G, tp_forward(prob, plus["x"], plus["Y"], plus["W"], src, dst, n))
              - np.vdot(G, tp_forward(prob, minus["x"], minus["Y"], minus["W"], src, dst, n))) / (2 * h)
        assert fd == pytest.approx(np.vdot(grad, d), rel=1e-11, abs=1e-11)


def test_scalar_channels_are_a_sparse_matmul():
    rng = np.random.default_rng(15)
    prob = TPProblem.build("3x0e", 0, "3x0e")
    n = 40
    E = 300
    src = rng.integers(0, n, E)
    dst = rng.integers(0, n, E)
    x = rng.standard_normal((n, 3))
    Y = rng.standard_normal((E, 1))
    W = rng.standard_normal((E, 3))
    out = tp_forward(prob, x, Y, W, src, dst, n)
    for u in range(3):
        A = sp.csr_matrix((W[:, u] * Y[:, 0], (dst, src)), shape=(n, n))
        np.testing.assert_allclose(out[:, u], A @ x[:, u], atol=1e-12)


def test_dot_product_path():
    rng = np.random.default_rng(16)
    prob = TPProblem.build("1x1o", 1, "1x0e")
    assert prob.paths == [(0, 1, 0)]
    n, E = 10, 60
    src, dst = rng.integers(0, n, E), rng.integers(0, n, E)
    x = rng.standard_normal((n, 3))
    Y = rng.standard_normal((E, 4))
    W = rng.standard_normal((E, 1))
    out = tp_forward(prob, x, Y, W, src, dst, n)
    ref = np.zeros(n)
    np.add.at(ref, dst, -W[:, 0] * (x[src] * Y[:, 1:4]).sum(1) / sqrt(3))
    np.testing.assert_allclose(out[:, 0], ref, atol=1e-12)


def test_edges_along_z_select_m2_zero():
    rng = np.random.default_rng(17)
    prob = TPProblem.build("2x0e+2x1o+2x2e", 2, "2x0e+2x1o+2x2e")
    n, E = 5, 12
    src, dst = rng.integers(0, n, E), rng.integers(0, n, E)
    x = rng.standard_normal((n, prob.dim_in))
    Y = sh_real(2, np.tile([0.0, 0.0, 2.5], (E, 1)))
    W = rng.standard_normal((E, prob.weight_numel))
    out = tp_forward(prob, x, Y, W, src, dst, n)
    ref = np.zeros_like(out)
    for p, (s1, l2, s3) in enumerate(prob.paths):
        l1, _, l3 = prob.path_ls(p)
        Cz = cg_real(l1, l2, l3)[:, l2, :] * sqrt(2 * l2 + 1)    # column m2 = 0
        xs = x[src][:, prob.irreps_in.slice(s1)].reshape(E, 2, 2 * l1 + 1)
        msg = np.einsum("eui,ik,eu->euk", xs, Cz, W[:, prob.weight_offsets[p]:prob.weight_offsets[p] + 2])
        np.add.at(ref[:, prob.irreps_out.slice(s3)], dst, msg.reshape(E, -1))
    np.testing.assert_allclose(out, ref, atol=1e-12)


def test_irreps_errors():
    with pytest.raises(ValueError):
        TPProblem.build("4x1q", 1, "4x1o")
    with pytest.raises(ValueError):
        TPProblem.build("4x0e", 1, "8x1o")     # uvu needs equal multiplicities
    with pytest.raises(ValueError):
        TPProblem.build("", 1, "1x0e")
    assert TPProblem.build("1x0e", 1, "1x2e").paths == []
