"""SO(2) convolution (oracle; test infrastructure).

The TrimSO(2) page (Abstract) describes SO(2)-convolution interatomic
potentials: a representation transformation around dense matrix
multiplications, which TrimSO(2) fuses as rotation on gather and inverse
rotation on reduction.  The page prints no formula; the plainest reading, the
one written out here, is:

  * every edge e (src j, dst i, vector r_e = pos[j] - pos[i]) has a frame
    rotation R_e, a proper rotation with R_e r_hat_e = z_hat;
  * the neighbour's features are rotated into that frame block by block,
    x~[l] = D^l(R_e) x[j, l] (per channel), D^l the real Wigner matrix with
    Y_l(R v) = D^l(R) Y_l(v) for the real harmonics of sh.py;
  * in the edge frame a linear map that commutes with rotations about z mixes
    degrees and channels at each |m| separately:
        m = 0:  y~_0  = A_0 X_0
        m > 0:  y~_+m = A_m X_+m - B_m X_-m,   y~_-m = B_m X_+m + A_m X_-m
    with X_+-m the vector of x~[l][c][+-m] over l = m..L (l major) and
    channels c, and A_m, B_m shared by all edges (the dense matmuls);
  * the result is rotated back and summed into the destination,
        out[i, l] += D^l(R_e)^T y~[l].

The map at |m| > 0 is complex multiplication by (A_m + i B_m) on
X_+m + i X_-m, which commutes with the 2x2 rotation by m*alpha that a z
rotation applies to each (+m, -m) pair, so the output does not depend on
which R_e is chosen among those taking r_hat to z_hat.  Activations, radial
modulation of the maps and a truncation of m are left out (the abstract
names no such detail for the convolution itself).

Layouts (all row-major, fp64 here):
  x, out  [N][C (L+1)^2]   degree l at offset C l^2, stored [C][2l+1]
  D       [E][sum_l (2l+1)^2]   block l at offset sum_{k<l} (2k+1)^2, [m][n]
  weights A_0, A_1, B_1, ..., A_L, B_L, each [K_m][K_m] (out, in) with
          K_m = (L+1-m) C and index (l-m) C + c.

R_e (the Rodrigues rotation about r_hat x z_hat by the angle between them;
identity for a zero vector or r_hat = z_hat, diag(1,-1,-1) for r_hat = -z_hat)
and D^l are fixed definitions so that D itself can be compared; the
convolution's output does not depend on that choice.
"""

from __future__ import annotations

import numpy as np

from .sh import sh_real


# ------------------------------------------------------------------ frames
def edge_rotation(vec: np.ndarray) -> np.ndarray:
    """[E,3,3] proper rotations with R r_hat = z_hat (Rodrigues' formula)."""
    vec = np.asarray(vec, dtype=np.float64).reshape(-1, 3)
    R = np.zeros((len(vec), 3, 3))
    for e, v in enumerate(vec):
        r = np.linalg.norm(v)
        if r == 0.0:
            R[e] = np.eye(3)
            continue
        u = v / r
        axis = np.cross(u, [0.0, 0.0, 1.0])          # (u_y, -u_x, 0)
        s = np.linalg.norm(axis)
        c = u[2]
        if s == 0.0:
            R[e] = np.eye(3) if c > 0 else np.diag([1.0, -1.0, -1.0])
            continue
        k = axis / s
        K = np.array([[0.0, -k[2], k[1]], [k[2], 0.0, -k[0]], [-k[1], k[0], 0.0]])
        R[e] = np.eye(3) + s * K + (1.0 - c) * (K @ K)  # angle theta: sin = s, cos = c
    return R


def sphere_quadrature(degree: int):
    """Points [K,3] and weights [K] (summing to 4 pi) that integrate every
    polynomial of total degree <= `degree` over the unit sphere exactly:
    Gauss-Legendre in z times equispaced azimuths."""
    nz = degree // 2 + 1
    nphi = degree + 1
    z, wz = np.polynomial.legendre.leggauss(nz)
    phi = 2.0 * np.pi * np.arange(nphi) / nphi
    zz, pp = np.meshgrid(z, phi, indexing="ij")
    rho = np.sqrt(1.0 - zz ** 2)
    pts = np.stack([rho * np.cos(pp), rho * np.sin(pp), zz], axis=-1).reshape(-1, 3)
    w = (wz[:, None] * np.full(nphi, 2.0 * np.pi / nphi)[None, :]).reshape(-1)
    return pts, w


def wigner_D(lmax: int, R: np.ndarray) -> list:
    """Real Wigner matrices D^l(R), l = 0..lmax, each [E, 2l+1, 2l+1], from
    their definition as the matrix of v -> Y_l(R v) in the basis Y_l:
        D^l[m, n] = (1/4 pi) integral over the sphere of Y_lm(R v) Y_ln(v)
    (the component-normalised harmonics are orthonormal under (1/4 pi) dOmega),
    evaluated with a quadrature exact for the degree-2l integrand."""
    R = np.asarray(R, dtype=np.float64).reshape(-1, 3, 3)
    pts, w = sphere_quadrature(2 * lmax)
    Yv = sh_real(lmax, pts)                                   # [K, (L+1)^2]
    out = []
    RY = sh_real(lmax, np.einsum("eab,kb->eka", R, pts))      # Y(R v_k)  [E, K, (L+1)^2]
    for l in range(lmax + 1):
        sl = slice(l * l, (l + 1) ** 2)
        out.append(np.einsum("k,ekm,kn->emn", w, RY[:, :, sl], Yv[:, sl]) / (4.0 * np.pi))
    return out


def pack_D(blocks: list) -> np.ndarray:
    """[E, sum (2l+1)^2] from the per-l blocks (row-major [m][n])."""
    return np.concatenate([b.reshape(b.shape[0], int(np.prod(b.shape[1:]))) for b in blocks], axis=1)


def unpack_D(D: np.ndarray, lmax: int) -> list:
    D = np.asarray(D, dtype=np.float64)
    out, off = [], 0
    for l in range(lmax + 1):
        n = 2 * l + 1
        out.append(D[:, off:off + n * n].reshape(-1, n, n))
        off += n * n
    return out


def edge_wigner(lmax: int, vec: np.ndarray) -> np.ndarray:
    """Packed D(R_e) for every edge vector: [E, sum (2l+1)^2]."""
    return pack_D(wigner_D(lmax, edge_rotation(vec)))


# ------------------------------------------------------------------ layout
def weight_blocks(lmax: int, C: int):
    """[(name, m, offset, K_m)] in storage order A_0, A_1, B_1, ..., A_L, B_L."""
    out, off = [], 0
    for m in range(lmax + 1):
        K = (lmax + 1 - m) * C
        out.append(("A", m, off, K))
        off += K * K
        if m > 0:
            out.append(("B", m, off, K))
            off += K * K
    return out


def weight_numel(lmax: int, C: int) -> int:
    return sum(K * K for _, _, _, K in weight_blocks(lmax, C))


def _maps(lmax, C, weights):
    weights = np.asarray(weights, dtype=np.float64)
    A, B = {}, {}
    for name, m, off, K in weight_blocks(lmax, C):
        (A if name == "A" else B)[m] = weights[off:off + K * K].reshape(K, K)
    return A, B


def _split(x, lmax, C):
    """[n, C (L+1)^2] -> list over l of [n, C, 2l+1]."""
    return [x[:, C * l * l:C * (l + 1) ** 2].reshape(len(x), C, 2 * l + 1) for l in range(lmax + 1)]


def _join(blocks):
    return np.concatenate([b.reshape(b.shape[0], int(np.prod(b.shape[1:]))) for b in blocks], axis=1)


def _gather_m(xt, lmax, m, sign):
    """X_{sign*m}: [n, K_m] over (l = m..L, c) of the rotated blocks."""
    return np.concatenate([xt[l][:, :, l + sign * m] for l in range(m, lmax + 1)], axis=1)


def _scatter_m(yt, lmax, C, m, sign, vals):
    for l in range(m, lmax + 1):
        yt[l][:, :, l + sign * m] = vals[:, (l - m) * C:(l - m + 1) * C]


def _so2_apply(xt, lmax, C, A, B, adjoint=False):
    """The per-|m| maps on rotated blocks (list over l of [n, C, 2l+1])."""
    n = len(xt[0])
    yt = [np.zeros((n, C, 2 * l + 1)) for l in range(lmax + 1)]
    for m in range(lmax + 1):
        a = A[m].T if adjoint else A[m]
        if m == 0:
            _scatter_m(yt, lmax, C, 0, 0, _gather_m(xt, lmax, 0, 0) @ a.T)
            continue
        b = -B[m].T if adjoint else B[m]           # adjoint of [[A,-B],[B,A]] is [[A^T,B^T],[-B^T,A^T]]
        xp, xm = _gather_m(xt, lmax, m, +1), _gather_m(xt, lmax, m, -1)
        _scatter_m(yt, lmax, C, m, +1, xp @ a.T - xm @ b.T)
        _scatter_m(yt, lmax, C, m, -1, xp @ b.T + xm @ a.T)
    return yt


def _rotate(blocks, Dl, transpose=False):
    """Per edge and channel: D^l v (or D^l^T v)."""
    spec = "emn,ecm->ecn" if transpose else "emn,ecn->ecm"
    return [np.einsum(spec, Dl[l], blocks[l]) for l in range(len(blocks))]


# ------------------------------------------------------------------ operator
def so2_forward(lmax, C, x, D, weights, src, dst, n_nodes):
    """out[i] = sum_{e: dst=i} D_e^T SO2(D_e x[src e])."""
    x = np.asarray(x, dtype=np.float64)
    src, dst = np.asarray(src, np.int64), np.asarray(dst, np.int64)
    A, B = _maps(lmax, C, weights)
    Dl = unpack_D(D, lmax)
    xt = _rotate(_split(x[src], lmax, C), Dl)
    yt = _so2_apply(xt, lmax, C, A, B)
    msg = _join(_rotate(yt, Dl, transpose=True))
    out = np.zeros((n_nodes, C * (lmax + 1) ** 2))
    np.add.at(out, dst, msg)
    return out


def so2_backward(lmax, C, x, D, weights, G, src, dst, n_nodes):
    """Gradients of <G, so2_forward(...)>: (grad_x [N, C(L+1)^2], grad_weights
    in the weights' layout).  With g~ = D_e G[dst e] and x~ = D_e x[src e]:
        grad_x[j]  = sum_{e: src=j} D_e^T SO2^T(g~)
        grad_A_0   = sum_e g~_0 X_0^T
        grad_A_m   = sum_e g~_+m X_+m^T + g~_-m X_-m^T
        grad_B_m   = sum_e g~_-m X_+m^T - g~_+m X_-m^T."""
    x = np.asarray(x, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    src, dst = np.asarray(src, np.int64), np.asarray(dst, np.int64)
    A, B = _maps(lmax, C, weights)
    Dl = unpack_D(D, lmax)
    xt = _rotate(_split(x[src], lmax, C), Dl)
    gt = _rotate(_split(G[dst], lmax, C), Dl)
    dxt = _so2_apply(gt, lmax, C, A, B, adjoint=True)
    grad_x = np.zeros((n_nodes, C * (lmax + 1) ** 2))
    np.add.at(grad_x, src, _join(_rotate(dxt, Dl, transpose=True)))
    gw = np.zeros(weight_numel(lmax, C))
    for name, m, off, K in weight_blocks(lmax, C):
        if m == 0:
            blk = _gather_m(gt, lmax, 0, 0).T @ _gather_m(xt, lmax, 0, 0)
        else:
            gp, gm = _gather_m(gt, lmax, m, +1), _gather_m(gt, lmax, m, -1)
            xp, xm = _gather_m(xt, lmax, m, +1), _gather_m(xt, lmax, m, -1)
            blk = gp.T @ xp + gm.T @ xm if name == "A" else gm.T @ xp - gp.T @ xm
        gw[off:off + K * K] = blk.reshape(-1)
    return grad_x, gw


def so2_weight_grad_entries(lmax, C, x, D, G, src, dst, idx):
    """Selected entries of so2_backward's grad_weights (flat indices idx into
    the weights' layout), each evaluated from its definition over all edges.
    With o = (lo - m) C + co and i = (li - m) C + ci the block's row and
    column, g~ = D_e G[dst e] and x~ = D_e x[src e]:
        A_0[o, i] = sum_e g~[lo][co][0] x~[li][ci][0]
        A_m[o, i] = sum_e g~[lo][co][+m] x~[li][ci][+m] + g~[lo][co][-m] x~[li][ci][-m]
        B_m[o, i] = sum_e g~[lo][co][-m] x~[li][ci][+m] - g~[lo][co][+m] x~[li][ci][-m]
    (m indexed -l..l).  Only the one channel block of G and of x that the
    entry touches is rotated, so an entry costs O(E) and any entry can be
    checked at any graph size."""
    x = np.asarray(x, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    src, dst = np.asarray(src, np.int64), np.asarray(dst, np.int64)
    Dl = unpack_D(D, lmax)
    blocks = weight_blocks(lmax, C)

    def rotated(V, nodes, l, c, mm):
        cols = V[:, C * l * l + c * (2 * l + 1):C * l * l + (c + 1) * (2 * l + 1)][nodes]   # [E, 2l+1]
        return np.einsum("en,en->e", Dl[l][:, l + mm, :], cols)

    out = np.zeros(len(idx))
    for t, j in enumerate(idx):
        name, m, off, K = next(b for b in blocks if b[2] <= j < b[2] + b[3] * b[3])
        o, i = divmod(int(j) - off, K)
        lo, co, li, ci = m + o // C, o % C, m + i // C, i % C
        if m == 0:
            out[t] = rotated(G, dst, lo, co, 0) @ rotated(x, src, li, ci, 0)
            continue
        gp, gm = rotated(G, dst, lo, co, m), rotated(G, dst, lo, co, -m)
        xp, xm = rotated(x, src, li, ci, m), rotated(x, src, li, ci, -m)
        out[t] = gp @ xp + gm @ xm if name == "A" else gm @ xp - gp @ xm
    return out


def so2_double_backward(lmax, C, x, D, weights, G, ggx, ggw, src, dst, n_nodes):
    """Gradients of L2 = <ggx, grad_x> + <ggw, grad_w>, where (grad_x, grad_w)
    = so2_backward(x, weights, G), with respect to x, the weights and G (the
    frames D held fixed).  The convolution f(x; w) is linear in x and in w
    separately, and grad_x = f(.; w)^T G, grad_w = the map gradient of (x, G),
    so
        L2 = <f(ggx; w), G> + <f(x; ggw), G>
    and
        grad_G = f(ggx; w) + f(x; ggw)
        grad_x = f(.; ggw)^T G         (the backward's grad_x with ggw for w)
        grad_w = map gradient of (ggx, G)  (the backward's grad_w with ggx for x).
    ggx or ggw may be None (zero).  Returns (grad_x, grad_w, grad_G)."""
    x = np.asarray(x, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    d = C * (lmax + 1) ** 2
    nw = weight_numel(lmax, C)
    grad_G = np.zeros((n_nodes, d))
    grad_x = np.zeros((n_nodes, d))
    grad_w = np.zeros(nw)
    if ggx is not None:
        grad_G += so2_forward(lmax, C, ggx, D, weights, src, dst, n_nodes)
        grad_w = so2_backward(lmax, C, ggx, D, weights, G, src, dst, n_nodes)[1]
    if ggw is not None:
        grad_G += so2_forward(lmax, C, x, D, ggw, src, dst, n_nodes)
        grad_x = so2_backward(lmax, C, x, D, ggw, G, src, dst, n_nodes)[0]
    return grad_x, grad_w, grad_G


# ------------------------------------------------- gradient through the frames
def so2_frames_backward(lmax, C, x, D, weights, G, src, dst, n_nodes):
    """grad_D [E, sum (2l+1)^2]: the gradient of <G, so2_forward(...)> with
    respect to each edge's Wigner blocks.  D_e enters twice, in the rotation
    on gather and in the inverse rotation, so with x~ = D_e x[src],
    y~ = SO2(x~), g~ = D_e G[dst] and dx~ = SO2^T(g~):
        grad_D^l[m][n] = sum_c dx~[l][c][m] x[src][l][c][n] + y~[l][c][m] G[dst][l][c][n]."""
    x = np.asarray(x, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    src, dst = np.asarray(src, np.int64), np.asarray(dst, np.int64)
    A, B = _maps(lmax, C, weights)
    Dl = unpack_D(D, lmax)
    xs, gd = _split(x[src], lmax, C), _split(G[dst], lmax, C)
    yt = _so2_apply(_rotate(xs, Dl), lmax, C, A, B)
    dxt = _so2_apply(_rotate(gd, Dl), lmax, C, A, B, adjoint=True)
    return pack_D([np.einsum("ecm,ecn->emn", dxt[l], xs[l]) + np.einsum("ecm,ecn->emn", yt[l], gd[l])
                   for l in range(lmax + 1)])


def _rotation_of(v):
    """edge_rotation's Rodrigues formula for one vector, written with plain
    arithmetic only (so that it also runs on complex inputs)."""
    r = np.sqrt(v[0] * v[0] + v[1] * v[1] + v[2] * v[2])
    u = v / r
    s = np.sqrt(u[0] * u[0] + u[1] * u[1])
    c = u[2]
    k = np.array([u[1] / s, -u[0] / s, 0.0 * s])
    K = np.array([[0.0 * s, -k[2], k[1]], [k[2], 0.0 * s, -k[0]], [-k[1], k[0], 0.0 * s]])
    return np.eye(3) + s * K + (1.0 - c) * (K @ K)


def rotations_backward(lmax, vec, grad_D):
    """grad_vec [E, 3] = sum over blocks of grad_D . dD/dvec for D = edge_wigner(lmax, vec).
    dD^l[m][n]/dR = (1/4 pi) sum_k w_k grad Y_lm(R p_k) p_k^T Y_ln(p_k) over the
    quadrature of wigner_D (the harmonics' Jacobian from forces.sh_and_jacobian;
    R stays a rotation, so only the tangential part of grad Y enters), and
    dR/dvec by the complex step on the Rodrigues formula (exact to rounding,
    no subtraction).  Zero vectors and vectors along the z axis, where the
    frame is set by convention, get zero."""
    from .forces import sh_and_jacobian
    vec = np.asarray(vec, dtype=np.float64).reshape(-1, 3)
    Gl = unpack_D(grad_D, lmax)
    pts, w = sphere_quadrature(2 * lmax)
    Yp = sh_real(lmax, pts)                                   # [K, (L+1)^2]
    out = np.zeros((len(vec), 3))
    hstep = 1e-30
    for e, v in enumerate(vec):
        if np.hypot(v[0], v[1]) == 0.0:
            continue
        R = _rotation_of(v)
        dR = np.stack([_rotation_of(v + 1j * hstep * np.eye(3)[j]).imag / hstep for j in range(3)])  # [3, 3, 3]
        q = pts @ R.T                                         # R p_k
        _, J = sh_and_jacobian(lmax, q)                       # [K, (L+1)^2, 3]
        # dL/dR_ab = (1/4pi) sum_k w_k sum_{l,m,n} Gl[m][n] dY_lm/dq_a (q_k) p_kb Y_ln(p_k)
        T = np.zeros((len(pts), (lmax + 1) ** 2))             # T[k, lm] = sum_n Gl[m][n] Y_ln(p_k)
        for l in range(lmax + 1):
            sl = slice(l * l, (l + 1) ** 2)
            T[:, sl] = Yp[:, sl] @ Gl[l][e].T
        dLdq = np.einsum("k,km,kma->ka", w, T, J) / (4.0 * np.pi)   # [K, 3]
        dLdR = dLdq.T @ pts                                   # [3, 3]: sum_k dLdq[k, a] p_k[b]
        out[e] = np.einsum("ab,jab->j", dLdR, dR)
    return out


def rotations_jvp(lmax, vec, dvec):
    """dD [E, sum (2l+1)^2]: the directional derivative of edge_wigner(lmax, vec)
    along dvec (per edge), from the same quadrature as wigner_D,
        dD^l[m][n] = (1/4 pi) sum_k w_k (grad Y_lm(R p_k) . dR p_k) Y_ln(p_k),
    with dR = sum_j dvec_j dR/dvec_j by the complex step on the Rodrigues
    formula (as in rotations_backward).  Vectors along the z axis (the zero
    vector included), where the frame is set by convention, get zero."""
    from .forces import sh_and_jacobian
    vec = np.asarray(vec, dtype=np.float64).reshape(-1, 3)
    dvec = np.asarray(dvec, dtype=np.float64).reshape(-1, 3)
    pts, w = sphere_quadrature(2 * lmax)
    Yp = sh_real(lmax, pts)                                   # [K, (L+1)^2]
    out = np.zeros((len(vec), sum((2 * l + 1) ** 2 for l in range(lmax + 1))))
    hstep = 1e-30
    for e, v in enumerate(vec):
        if np.hypot(v[0], v[1]) == 0.0:
            continue
        R = _rotation_of(v)
        dR = _rotation_of(v + 1j * hstep * dvec[e]).imag / hstep   # [3, 3]
        q = pts @ R.T                                         # R p_k
        dq = pts @ dR.T                                       # dR p_k
        _, J = sh_and_jacobian(lmax, q)                       # [K, (L+1)^2, 3]
        dY = np.einsum("kma,ka->km", J, dq)                   # derivative of Y(R p_k) along dR
        blocks = []
        for l in range(lmax + 1):
            sl = slice(l * l, (l + 1) ** 2)
            blocks.append(np.einsum("k,km,kn->mn", w, dY[:, sl], Yp[:, sl]).reshape(-1) / (4.0 * np.pi))
        out[e] = np.concatenate(blocks)
    return out


def so2_frames_double_backward(lmax, C, x, D, weights, G, dD, src, dst, n_nodes, parts=False):
    """Gradients of S = <dD, so2_frames_backward(lmax, C, x, D, weights, G, ...)>
    with respect to x, the weights and G (the frames D held fixed): the mixed
    second derivatives that training on forces through the frames needs (dD
    is the frames' derivative along the force cotangent, rotations_jvp).
    grad_D_e = dx~ x^T + y~ g^T per block is linear in x, G and the maps, and
    moving the maps across each term,
        S = sum_e <dD_e g, SO2(D_e x)> + <D_e g, SO2(dD_e x)>
    (g = G[dst e], x = x[src e]), so
        grad_G[dst] += dD_e^T SO2(D_e x) + D_e^T SO2(dD_e x)
        grad_x[src] += D_e^T SO2^T(dD_e g) + dD_e^T SO2^T(D_e g)
        grad_w       = the map gradients of the pairs (dD_e g, D_e x) and
                       (D_e g, dD_e x), as in so2_backward.
    Returns (grad_x, grad_w, grad_G); with parts=True each is instead the
    pair of its two terms in the order written above (first the one with dD
    on the output side or on g), whose sum is the gradient.  The pair shows
    how much the two terms cancel: for frames' derivatives dD = Omega D with
    Omega antisymmetric they cancel exactly in the part of Omega that
    commutes with the SO(2) maps (the rotation about the edge axis)."""
    x = np.asarray(x, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    src, dst = np.asarray(src, np.int64), np.asarray(dst, np.int64)
    A, B = _maps(lmax, C, weights)
    Dl = unpack_D(D, lmax)
    Cl = unpack_D(dD, lmax)
    xs, gd = _split(x[src], lmax, C), _split(G[dst], lmax, C)
    xD, xC = _rotate(xs, Dl), _rotate(xs, Cl)
    gD, gC = _rotate(gd, Dl), _rotate(gd, Cl)
    d = C * (lmax + 1) ** 2
    gG1, gG2 = np.zeros((n_nodes, d)), np.zeros((n_nodes, d))
    np.add.at(gG1, dst, _join(_rotate(_so2_apply(xD, lmax, C, A, B), Cl, transpose=True)))
    np.add.at(gG2, dst, _join(_rotate(_so2_apply(xC, lmax, C, A, B), Dl, transpose=True)))
    gx1, gx2 = np.zeros((n_nodes, d)), np.zeros((n_nodes, d))
    np.add.at(gx1, src, _join(_rotate(_so2_apply(gC, lmax, C, A, B, adjoint=True), Dl, transpose=True)))
    np.add.at(gx2, src, _join(_rotate(_so2_apply(gD, lmax, C, A, B, adjoint=True), Cl, transpose=True)))
    gws = []
    for gt, xt in ((gC, xD), (gD, xC)):
        gw = np.zeros(weight_numel(lmax, C))
        for name, m, off, K in weight_blocks(lmax, C):
            if m == 0:
                blk = _gather_m(gt, lmax, 0, 0).T @ _gather_m(xt, lmax, 0, 0)
            else:
                gp, gm = _gather_m(gt, lmax, m, +1), _gather_m(gt, lmax, m, -1)
                xp, xm = _gather_m(xt, lmax, m, +1), _gather_m(xt, lmax, m, -1)
                blk = gp.T @ xp + gm.T @ xm if name == "A" else gm.T @ xp - gp.T @ xm
            gw[off:off + K * K] = blk.reshape(-1)
        gws.append(gw)
    if parts:
        return (gx1, gx2), (gws[0], gws[1]), (gG1, gG2)
    return gx1 + gx2, gws[0] + gws[1], gG1 + gG2
