"""Dense per-edge CGTP convolution: forward, backward and double backward (oracle; test infrastructure).

Definition (the plain reading of the "CGTP convolution" in the LunaTP abstract
and of the "tensor-product layer and its following reduce layer" in the FlashTP
summary, sections "Problem" and "Approach"; the pages print no formula).  For an
edge e with j = src(e), i = dst(e), a path p = (s1, l2, s3) with real CG tensor
C_p and a channel u:

  out[i,s3,u,m3] = sum_{e: dst=i} sum_{p -> s3} W[e,p,u] sum_{m1,m2} C_p[m1,m2,m3] x[j,s1,u,m1] Y[e,l2,m2]
  dx [j,s1,u,m1] = sum_{e: src=j} sum_{p <- s1} W[e,p,u] sum_{m2,m3} C_p[m1,m2,m3] Y[e,l2,m2] G[i,s3,u,m3]
  dY [e,l2,m2]   = sum_{p with l2} sum_u W[e,p,u] sum_{m1,m3} C_p[m1,m2,m3] x[j,s1,u,m1] G[i,s3,u,m3]
  dW [e,p,u]     = sum_{m1,m2,m3} C_p[m1,m2,m3] x[j,s1,u,m1] Y[e,l2,m2] G[i,s3,u,m3]

G is the supplied gradient of the loss with respect to out.  Everything is
evaluated in fp64 (inputs given in fp32 are upcast exactly), path by path, in
edge chunks, with np.add.at for the scatter-sum.  Layouts:

  x[N, D_in]   segments concatenated; segment s stored [mul_s][2 l_s + 1]
  Y[E, (L+1)^2] (l, m) at column l*l + l + m
  W[E, sum_p mul_p]  path p at columns [off_p, off_p + mul_p)
  out[N, D_out] like x.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List, Tuple

import numpy as np

from .cg import cg_real
from .irreps import Irreps, enumerate_paths, parse_irreps


@dataclass
class TPProblem:
    irreps_in: Irreps
    sh_lmax: int
    irreps_out: Irreps
    paths: List[Tuple[int, int, int]]
    weight_offsets: List[int]
    weight_numel: int

    @classmethod
    def build(cls, irreps_in: str, sh_lmax: int, irreps_out: str) -> "TPProblem":
        a, c = parse_irreps(irreps_in), parse_irreps(irreps_out)
        if sh_lmax < 0:
            raise ValueError("sh_lmax must be >= 0")
        paths = enumerate_paths(a, sh_lmax, c)
        offs, o = [], 0
        for s1, _, _ in paths:
            offs.append(o)
            o += a[s1].mul
        return cls(a, sh_lmax, c, paths, offs, o)

    @property
    def dim_in(self) -> int:
        return self.irreps_in.dim

    @property
    def dim_out(self) -> int:
        return self.irreps_out.dim

    @property
    def dim_sh(self) -> int:
        return (self.sh_lmax + 1) ** 2

    def path_ls(self, p: int) -> Tuple[int, int, int]:
        s1, l2, s3 = self.paths[p]
        return self.irreps_in[s1].l, l2, self.irreps_out[s3].l


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def _chunks(n: int, size: int):
    for a in range(0, n, size):
        yield a, min(n, a + size)


def tp_forward(prob: TPProblem, x, Y, W, src, dst, n_nodes: int, chunk: int = 8192) -> np.ndarray:
    x, Y, W = _f64(x), _f64(Y), _f64(W)
    src = np.asarray(src, dtype=np.int64)
    dst = np.asarray(dst, dtype=np.int64)
    E = src.shape[0]
    out = np.zeros((n_nodes, prob.dim_out))
    for p, (s1, l2, s3) in enumerate(prob.paths):
        l1, _, l3 = prob.path_ls(p)
        mul = prob.irreps_in[s1].mul
        C = cg_real(l1, l2, l3)
        sin, sout = prob.irreps_in.slice(s1), prob.irreps_out.slice(s3)
        wo = prob.weight_offsets[p]
        view = out[:, sout]
        for a, b in _chunks(E, chunk):
            xs = x[src[a:b], sin].reshape(b - a, mul, 2 * l1 + 1)
            ys = Y[a:b, l2 * l2:(l2 + 1) ** 2]
            w = W[a:b, wo:wo + mul]
            msg = np.einsum("eui,ej,ijk,eu->euk", xs, ys, C, w, optimize=True)
            np.add.at(view, dst[a:b], msg.reshape(b - a, -1))
    return out


def tp_backward(prob: TPProblem, x, Y, W, G, src, dst, n_nodes: int, chunk: int = 8192):
    """Returns (dx [N, D_in], dY [E, D_sh], dW [E, weight_numel])."""
    x, Y, W, G = _f64(x), _f64(Y), _f64(W), _f64(G)
    src = np.asarray(src, dtype=np.int64)
    dst = np.asarray(dst, dtype=np.int64)
    E = src.shape[0]
    dx = np.zeros((n_nodes, prob.dim_in))
    dY = np.zeros((E, prob.dim_sh))
    dW = np.zeros((E, prob.weight_numel))
    for p, (s1, l2, s3) in enumerate(prob.paths):
        l1, _, l3 = prob.path_ls(p)
        mul = prob.irreps_in[s1].mul
        C = cg_real(l1, l2, l3)
        sin, sout = prob.irreps_in.slice(s1), prob.irreps_out.slice(s3)
        wo = prob.weight_offsets[p]
        dxv = dx[:, sin]
        for a, b in _chunks(E, chunk):
            xs = x[src[a:b], sin].reshape(b - a, mul, 2 * l1 + 1)
            gs = G[dst[a:b], sout].reshape(b - a, mul, 2 * l3 + 1)
            ys = Y[a:b, l2 * l2:(l2 + 1) ** 2]
            w = W[a:b, wo:wo + mul]
            dW[a:b, wo:wo + mul] = np.einsum("eui,ej,ijk,euk->eu", xs, ys, C, gs, optimize=True)
            dxe = np.einsum("ej,ijk,euk,eu->eui", ys, C, gs, w, optimize=True)
            np.add.at(dxv, src[a:b], dxe.reshape(b - a, -1))
            dY[a:b, l2 * l2:(l2 + 1) ** 2] += np.einsum("eui,ijk,euk,eu->ej", xs, C, gs, w, optimize=True)
    return dx, dY, dW


def tp_double_backward(prob: TPProblem, x, Y, W, G, ggx, ggY, ggW, src, dst, n_nodes: int, chunk: int = 8192):
    """Gradients of L2 = <ggx, dx> + <ggY, dY> + <ggW, dW>, where (dx, dY, dW) is
    tp_backward(x, Y, W, G), with respect to x, Y, W and G.

    This is the double backward of the convolution: the second derivatives a
    force-trained potential needs (the FlashTP page lists an fp64 l_max = 4
    double-backward kernel result under "Key results"; the LunaTP and TrimSO(2)
    abstracts name higher-order derivatives / double backward as part of
    training).  The pages give no formula; written out from the definitions
    in this module's header, with a = ggx, b = ggY, c = ggW:

      L2 = sum_e sum_p sum_u sum_{m1,m2,m3} C_p[m1,m2,m3] G[i,s3,u,m3] *
             ( W[e,p,u] a[j,s1,u,m1] Y[e,l2,m2]
             + W[e,p,u] x[j,s1,u,m1] b[e,l2,m2]
             + c[e,p,u] x[j,s1,u,m1] Y[e,l2,m2] )

    and each gradient is the plain partial derivative of that sum:

      gG[i,s3,u,m3] = sum_{e: dst=i} sum_{p -> s3} sum_{m1,m2} C (W a Y + W x b + c x Y)
      gx[j,s1,u,m1] = sum_{e: src=j} sum_{p <- s1} sum_{m2,m3} C G (W b + c Y)
      gY[e,l2,m2]   = sum_{p with l2} sum_u sum_{m1,m3} C G (W a + c x)
      gW[e,p,u]     = sum_{m1,m2,m3} C G (a Y + x b)

    Any of ggx, ggY, ggW may be None (zero).  Returns (gx [N, D_in],
    gY [E, D_sh], gW [E, weight_numel], gG [N, D_out]).
    """
    x, Y, W, G = _f64(x), _f64(Y), _f64(W), _f64(G)
    E = np.asarray(src).shape[0]
    a = np.zeros_like(x) if ggx is None else _f64(ggx)
    b = np.zeros_like(Y) if ggY is None else _f64(ggY)
    c = np.zeros_like(W) if ggW is None else _f64(ggW)
    src = np.asarray(src, dtype=np.int64)
    dst = np.asarray(dst, dtype=np.int64)
    gx = np.zeros((n_nodes, prob.dim_in))
    gY = np.zeros((E, prob.dim_sh))
    gW = np.zeros((E, prob.weight_numel))
    gG = np.zeros((n_nodes, prob.dim_out))
    for p, (s1, l2, s3) in enumerate(prob.paths):
        l1, _, l3 = prob.path_ls(p)
        mul = prob.irreps_in[s1].mul
        C = cg_real(l1, l2, l3)
        sin, sout = prob.irreps_in.slice(s1), prob.irreps_out.slice(s3)
        wo = prob.weight_offsets[p]
        ysl = slice(l2 * l2, (l2 + 1) ** 2)
        gxv, gGv = gx[:, sin], gG[:, sout]
        for lo, hi in _chunks(E, chunk):
            n = hi - lo
            xs = x[src[lo:hi], sin].reshape(n, mul, 2 * l1 + 1)
            as_ = a[src[lo:hi], sin].reshape(n, mul, 2 * l1 + 1)
            gs = G[dst[lo:hi], sout].reshape(n, mul, 2 * l3 + 1)
            ys, bs = Y[lo:hi, ysl], b[lo:hi, ysl]
            w, cw = W[lo:hi, wo:wo + mul], c[lo:hi, wo:wo + mul]
            msg = (np.einsum("eui,ej,ijk,eu->euk", as_, ys, C, w, optimize=True)
                   + np.einsum("eui,ej,ijk,eu->euk", xs, bs, C, w, optimize=True)
                   + np.einsum("eui,ej,ijk,eu->euk", xs, ys, C, cw, optimize=True))
            np.add.at(gGv, dst[lo:hi], msg.reshape(n, -1))
            gxe = (np.einsum("ej,ijk,euk,eu->eui", bs, C, gs, w, optimize=True)
                   + np.einsum("ej,ijk,euk,eu->eui", ys, C, gs, cw, optimize=True))
            np.add.at(gxv, src[lo:hi], gxe.reshape(n, -1))
            gY[lo:hi, ysl] += (np.einsum("eui,ijk,euk,eu->ej", as_, C, gs, w, optimize=True)
                               + np.einsum("eui,ijk,euk,eu->ej", xs, C, gs, cw, optimize=True))
            gW[lo:hi, wo:wo + mul] = (np.einsum("eui,ej,ijk,euk->eu", as_, ys, C, gs, optimize=True)
                                      + np.einsum("eui,ej,ijk,euk->eu", xs, bs, C, gs, optimize=True))
    return gx, gY, gW, gG
