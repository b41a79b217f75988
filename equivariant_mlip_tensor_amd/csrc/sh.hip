// sh.hip -- the step upstream of the convolution on gfx950 as separate
// streaming kernels: edge spherical harmonics from edge vectors, their
// gradient, and the position gradient (forces).  The convolution kernels can
// also evaluate the harmonics of their edges themselves (tpconv_forward_vec,
// tpconv_backward_vec); both use the device functions of sh_eval.hpp, so the
// values agree.
//
// Also the SO(2) convolution's edge frames: the real Wigner blocks of each
// edge's frame rotation (k_so2_wigner) and their gradient with respect to
// the edge vector (k_so2_wigner_backward), both from an exact sphere
// quadrature of the same harmonics.
//
// Arithmetic is fp64 for both data types (fp32 inputs are widened, results
// rounded once on store): the gradient is the small tangential remainder of
// grad S - l S u, so fp32 evaluation loses ~10x its working precision, and
// these kernels are bound by memory traffic, where fp64 (full rate on CDNA)
// costs nothing measurable.
#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>

#include "sh_eval.hpp"
#include "tp_common.hpp"

namespace tpconv {
namespace {

using namespace shx;

template <typename T, int L>
__global__ __launch_bounds__(256) void k_sh(int64_t n, const T* __restrict__ vec, T* __restrict__ Y) {
  constexpr int D = (L + 1) * (L + 1);
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  const T* v = vec + 3 * e;
  T* yr = Y + e * D;
  sh_values<L>(double(v[0]), double(v[1]), double(v[2]), [&](int k, double val) { yr[k] = T(val); });
}

// grad_vec[e] = sum_lm grad_Y[e, lm] dY_lm/dvec (sh_vec_grad)
template <typename T, int L>
__global__ __launch_bounds__(256) void k_sh_backward(int64_t n, const T* __restrict__ vec, const T* __restrict__ gY,
                                                     T* __restrict__ gvec) {
  constexpr int D = (L + 1) * (L + 1);
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  const T* v = vec + 3 * e;
  const T* g = gY + e * D;
  double gx, gy, gz;
  sh_vec_grad<L>(double(v[0]), double(v[1]), double(v[2]), [&](int k) { return double(g[k]); }, gx, gy, gz);
  T* out = gvec + 3 * e;
  out[0] = T(gx);
  out[1] = T(gy);
  out[2] = T(gz);
}

// grad_pos[j] = sum over edges leaving j of grad_vec - sum over edges entering j:
// one wavefront per node walks the node's row in both CSR views, lane-strided,
// then a fixed butterfly; same order every run.
template <typename T>
__global__ __launch_bounds__(256) void k_pos_backward(int64_t n_nodes, const int32_t* __restrict__ src_row,
                                                      const int32_t* __restrict__ src_eid,
                                                      const int32_t* __restrict__ dst_row,
                                                      const int32_t* __restrict__ dst_eid, const T* __restrict__ gv,
                                                      T* __restrict__ gpos) {
  using A = double;
  const int lane = threadIdx.x & 63;
  const int64_t node = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (node >= n_nodes) return;  // wave-uniform
  A s0 = 0, s1 = 0, s2 = 0;
  for (int k = src_row[node] + lane; k < src_row[node + 1]; k += 64) {
    const T* p = gv + 3 * (int64_t)src_eid[k];
    s0 += A(p[0]);
    s1 += A(p[1]);
    s2 += A(p[2]);
  }
  for (int k = dst_row[node] + lane; k < dst_row[node + 1]; k += 64) {
    const T* p = gv + 3 * (int64_t)dst_eid[k];
    s0 -= A(p[0]);
    s1 -= A(p[1]);
    s2 -= A(p[2]);
  }
  for (int off = 32; off >= 1; off >>= 1) {
    s0 += __shfl_xor(s0, off, 64);
    s1 += __shfl_xor(s1, off, 64);
    s2 += __shfl_xor(s2, off, 64);
  }
  if (lane == 0) {
    gpos[3 * node] = T(s0);
    gpos[3 * node + 1] = T(s1);
    gpos[3 * node + 2] = T(s2);
  }
}

// Edge frames for the SO(2) convolution.  R_e is the proper rotation about
// u x z_hat through the angle between u = r / |r| and z_hat (Rodrigues'
// formula), so R_e u = z_hat; the identity for a zero vector or u = z_hat and
// diag(1, -1, -1) for u = -z_hat.  Its real Wigner blocks,
//   D^l[m][n] = (1 / 4 pi) integral over the sphere of Y_lm(R v) Y_ln(v),
// the matrix of v -> Y_l(R v) in the basis Y_l, come from a product rule
// that is exact for the degree-2l integrand: L + 1 Gauss-Legendre nodes in z
// (closed forms) times 2L + 1 equispaced azimuths.  fp64 throughout.
__device__ __forceinline__ void gauss_legendre(int n, int i, double& x, double& w) {
  // nodes ascending; the closed forms for n <= 5
  switch (n) {
    case 1: x = 0.0; w = 2.0; return;
    case 2: x = (i == 0 ? -1.0 : 1.0) / sqrt(3.0); w = 1.0; return;
    case 3: {
      const double a = sqrt(0.6);
      x = i == 0 ? -a : (i == 1 ? 0.0 : a);
      w = i == 1 ? 8.0 / 9.0 : 5.0 / 9.0;
      return;
    }
    case 4: {
      const double t = 2.0 / 7.0 * sqrt(6.0 / 5.0);
      const double inner = sqrt(3.0 / 7.0 - t), outer = sqrt(3.0 / 7.0 + t);
      const double wi = (18.0 + sqrt(30.0)) / 36.0, wo = (18.0 - sqrt(30.0)) / 36.0;
      const double xs[4] = {-outer, -inner, inner, outer}, ws[4] = {wo, wi, wi, wo};
      x = xs[i];
      w = ws[i];
      return;
    }
    default: {
      const double t = 2.0 * sqrt(10.0 / 7.0);
      const double inner = sqrt(5.0 - t) / 3.0, outer = sqrt(5.0 + t) / 3.0;
      const double wi = (322.0 + 13.0 * sqrt(70.0)) / 900.0, wo = (322.0 - 13.0 * sqrt(70.0)) / 900.0;
      const double xs[5] = {-outer, -inner, 0.0, inner, outer}, ws[5] = {wo, wi, 128.0 / 225.0, wi, wo};
      x = xs[i];
      w = ws[i];
      return;
    }
  }
}

// The frames' quadrature, the same for every edge, built once per block in
// LDS: point k = (iz, ip), its weight w_k / (4 pi) and the solid harmonics
// there.
template <int L>
struct FrameQuad {
  static constexpr int NZ = L + 1, NP = 2 * L + 1, NQ = NZ * NP, NS = (L + 1) * (L + 1);
  double p[NQ][3];
  double w[NQ];
  double S[NQ][NS];
};

template <int L>
__device__ __forceinline__ void frame_quad_fill(FrameQuad<L>& Q) {
  using F = FrameQuad<L>;
  for (int k = threadIdx.x; k < F::NQ; k += blockDim.x) {
    const int iz = k / F::NP, ip = k - iz * F::NP;
    double z, wz, sp, cp;
    gauss_legendre(F::NZ, iz, z, wz);
    const double rho = sqrt(fmax(0.0, 1.0 - z * z));
    sincos(2.0 * M_PI * ip / F::NP, &sp, &cp);
    Q.p[k][0] = rho * cp;
    Q.p[k][1] = rho * sp;
    Q.p[k][2] = z;
    Q.w[k] = wz / (2.0 * F::NP);  // (wz * 2 pi / NP) / (4 pi)
    double S[F::NS];
    solid_harmonics<L, double, PlainOps<double>>(rho * cp, rho * sp, z, 1.0, 1.0, S);
    for (int q = 0; q < F::NS; ++q) Q.S[k][q] = S[q];
  }
  __syncthreads();
}

template <typename T, int L>
__global__ __launch_bounds__(64) void k_so2_wigner(int64_t n, const T* __restrict__ vec, T* __restrict__ D) {
  constexpr int NS = (L + 1) * (L + 1);
  constexpr int ND = (L + 1) * (2 * L + 1) * (2 * L + 3) / 3;
  __shared__ FrameQuad<L> Q;
  frame_quad_fill<L>(Q);
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  double ux, uy, uz;
  const double r = load_unit(vec + 3 * e, ux, uy, uz);
  double R[3][3] = {{1.0, 0.0, 0.0}, {0.0, 1.0, 0.0}, {0.0, 0.0, 1.0}};
  if (r > 0.0) {
    const double sn = sqrt(ux * ux + uy * uy), cs = uz;
    if (sn == 0.0) {
      if (cs < 0.0) R[1][1] = R[2][2] = -1.0;
    } else {
      const double kx = uy / sn, ky = -ux / sn;  // unit axis u x z_hat / |u x z_hat|, kz = 0
      const double K[3][3] = {{0.0, 0.0, ky}, {0.0, 0.0, -kx}, {-ky, kx, 0.0}};
      for (int a = 0; a < 3; ++a)
        for (int b = 0; b < 3; ++b) {
          double k2 = 0.0;
          for (int q = 0; q < 3; ++q) k2 += K[a][q] * K[q][b];
          R[a][b] += sn * K[a][b] + (1.0 - cs) * k2;
        }
    }
  }
  double acc[ND];
  for (int q = 0; q < ND; ++q) acc[q] = 0.0;
  for (int k = 0; k < FrameQuad<L>::NQ; ++k) {
    {
      const double px = Q.p[k][0], py = Q.p[k][1], z = Q.p[k][2];
      const double qx = R[0][0] * px + R[0][1] * py + R[0][2] * z;
      const double qy = R[1][0] * px + R[1][1] * py + R[1][2] * z;
      const double qz = R[2][0] * px + R[2][1] * py + R[2][2] * z;
      const double* Sp = Q.S[k];
      double Sq[NS];
      solid_harmonics<L, double, PlainOps<double>>(qx, qy, qz, 1.0, 1.0, Sq);
      const double w = Q.w[k];
      sh_for<L + 1>([&](auto IL) {
        constexpr int l = IL, n2 = 2 * l + 1, off = l * (2 * l - 1) * (2 * l + 1) / 3;
        const double wl = w * n2;  // Y = sqrt(2l+1) S on the unit sphere
        sh_for<n2>([&](auto M) {
          const double a = wl * Sq[l * l + M];
          sh_for<n2>([&](auto N) { acc[off + M * n2 + N] += a * Sp[l * l + N]; });
        });
      });
    }
  }
  T* out = D + e * ND;
  for (int q = 0; q < ND; ++q) out[q] = T(acc[q]);
}

// The gradient through the frames: grad_vec[e] = sum_{l,m,n} grad_D[e]^l[m][n]
// dD^l[m][n]/dvec, differentiating the same quadrature,
//   dD^l[m][n]/dvec = sum_k w_k (2l+1) (dS_lm(R p_k)/dvec) S_ln(p_k),
// with dual numbers carrying d/dvec through the Rodrigues frame and the
// solid-harmonic recurrences at q_k = R p_k.  Vectors on the z axis (the
// zero vector included), where the frame is set by convention, get zero.
template <typename T>
__device__ __forceinline__ Dual<T> dsum(const Dual<T>& a, const Dual<T>& b) {
  return {a.v + b.v, a.dx + b.dx, a.dy + b.dy, a.dz + b.dz};
}
template <typename T>
__device__ __forceinline__ Dual<T> dsqrt(const Dual<T>& a) {
  const T v = sqrt(a.v), f = T(0.5) / v;
  return {v, a.dx * f, a.dy * f, a.dz * f};
}
template <typename T>
__device__ __forceinline__ Dual<T> ddiv(const Dual<T>& a, const Dual<T>& b) {
  const T iv = T(1) / b.v, q = a.v * iv;
  return {q, (a.dx - q * b.dx) * iv, (a.dy - q * b.dy) * iv, (a.dz - q * b.dz) * iv};
}

template <typename T, int L>
__global__ __launch_bounds__(64) void k_so2_wigner_backward(int64_t n, const T* __restrict__ vec,
                                                            const T* __restrict__ gD, T* __restrict__ gvec) {
  using D3 = Dual<double>;
  constexpr int NS = (L + 1) * (L + 1);
  constexpr int ND = (L + 1) * (2 * L + 1) * (2 * L + 3) / 3;
  __shared__ FrameQuad<L> Q;
  frame_quad_fill<L>(Q);
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  const double vx = vec[3 * e], vy = vec[3 * e + 1], vz = vec[3 * e + 2];
  T* o = gvec + 3 * e;
  if (vx == 0.0 && vy == 0.0) {
    o[0] = o[1] = o[2] = T(0);
    return;
  }
  const D3 X{vx, 1.0, 0.0, 0.0}, Yv{vy, 0.0, 1.0, 0.0}, Z{vz, 0.0, 0.0, 1.0};
  const D3 r = dsqrt(dsum(dsum(dmul(X, X), dmul(Yv, Yv)), dmul(Z, Z)));
  const D3 ux = ddiv(X, r), uy = ddiv(Yv, r), uz = ddiv(Z, r);
  const D3 sn = dsqrt(dsum(dmul(ux, ux), dmul(uy, uy)));
  const D3 kx = ddiv(uy, sn), ky = dscale(-1.0, ddiv(ux, sn));
  const D3 zero{0.0, 0.0, 0.0, 0.0};
  const D3 one_m_c = dlin(1.0, D3{1.0, 0.0, 0.0, 0.0}, -1.0, uz);
  const D3 K[3][3] = {{zero, zero, ky}, {zero, zero, dscale(-1.0, kx)}, {dscale(-1.0, ky), kx, zero}};
  D3 R[3][3];
  for (int a = 0; a < 3; ++a)
    for (int b = 0; b < 3; ++b) {
      D3 k2 = zero;
      for (int q = 0; q < 3; ++q) k2 = dsum(k2, dmul(K[a][q], K[q][b]));
      R[a][b] = dsum(dsum(D3{a == b ? 1.0 : 0.0, 0.0, 0.0, 0.0}, dmul(sn, K[a][b])), dmul(one_m_c, k2));
    }
  double g[ND];
  for (int q = 0; q < ND; ++q) g[q] = gD[e * ND + q];
  double gx = 0.0, gy = 0.0, gz = 0.0;
  for (int k = 0; k < FrameQuad<L>::NQ; ++k) {
    {
      const double p[3] = {Q.p[k][0], Q.p[k][1], Q.p[k][2]};
      D3 q[3];
      for (int a = 0; a < 3; ++a) q[a] = dsum(dsum(dscale(p[0], R[a][0]), dscale(p[1], R[a][1])), dscale(p[2], R[a][2]));
      const D3 q2 = dsum(dsum(dmul(q[0], q[0]), dmul(q[1], q[1])), dmul(q[2], q[2]));
      const double* Sp = Q.S[k];
      D3 Sq[NS];
      solid_harmonics<L, D3, DualOps<double>>(q[0], q[1], q[2], q2, D3{1.0, 0.0, 0.0, 0.0}, Sq);
      const double w = Q.w[k];
      sh_for<L + 1>([&](auto IL) {
        constexpr int l = IL, n2 = 2 * l + 1, off = l * (2 * l - 1) * (2 * l + 1) / 3;
        const double wl = w * n2;
        sh_for<n2>([&](auto M) {
          double t = 0.0;
          sh_for<n2>([&](auto N) { t += g[off + M * n2 + N] * Sp[l * l + N]; });
          t *= wl;
          const D3& sq = Sq[l * l + M];
          gx += t * sq.dx;
          gy += t * sq.dy;
          gz += t * sq.dz;
        });
      });
    }
  }
  o[0] = T(gx);
  o[1] = T(gy);
  o[2] = T(gz);
}

// The frames' directional derivative along dvec: the same dual numbers as
// the gradient above, contracted with dvec instead of with grad_D,
//   dD^l[m][n] = sum_k w_k (2l+1) (dvec . dS_lm(R p_k)/dvec) S_ln(p_k).
// Vectors on the z axis (the zero vector included) get zero.
template <typename T, int L>
__global__ __launch_bounds__(64) void k_so2_wigner_jvp(int64_t n, const T* __restrict__ vec,
                                                       const T* __restrict__ dvec, T* __restrict__ dD) {
  using D3 = Dual<double>;
  constexpr int NS = (L + 1) * (L + 1);
  constexpr int ND = (L + 1) * (2 * L + 1) * (2 * L + 3) / 3;
  __shared__ FrameQuad<L> Q;
  frame_quad_fill<L>(Q);
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  const double vx = vec[3 * e], vy = vec[3 * e + 1], vz = vec[3 * e + 2];
  T* o = dD + e * ND;
  if (vx == 0.0 && vy == 0.0) {
    for (int q = 0; q < ND; ++q) o[q] = T(0);
    return;
  }
  const double tx = dvec[3 * e], ty = dvec[3 * e + 1], tz = dvec[3 * e + 2];
  const D3 X{vx, 1.0, 0.0, 0.0}, Yv{vy, 0.0, 1.0, 0.0}, Z{vz, 0.0, 0.0, 1.0};
  const D3 r = dsqrt(dsum(dsum(dmul(X, X), dmul(Yv, Yv)), dmul(Z, Z)));
  const D3 ux = ddiv(X, r), uy = ddiv(Yv, r), uz = ddiv(Z, r);
  const D3 sn = dsqrt(dsum(dmul(ux, ux), dmul(uy, uy)));
  const D3 kx = ddiv(uy, sn), ky = dscale(-1.0, ddiv(ux, sn));
  const D3 zero{0.0, 0.0, 0.0, 0.0};
  const D3 one_m_c = dlin(1.0, D3{1.0, 0.0, 0.0, 0.0}, -1.0, uz);
  const D3 K[3][3] = {{zero, zero, ky}, {zero, zero, dscale(-1.0, kx)}, {dscale(-1.0, ky), kx, zero}};
  D3 R[3][3];
  for (int a = 0; a < 3; ++a)
    for (int b = 0; b < 3; ++b) {
      D3 k2 = zero;
      for (int q = 0; q < 3; ++q) k2 = dsum(k2, dmul(K[a][q], K[q][b]));
      R[a][b] = dsum(dsum(D3{a == b ? 1.0 : 0.0, 0.0, 0.0, 0.0}, dmul(sn, K[a][b])), dmul(one_m_c, k2));
    }
  double acc[ND];
  for (int q = 0; q < ND; ++q) acc[q] = 0.0;
  for (int k = 0; k < FrameQuad<L>::NQ; ++k) {
    {
      const double p[3] = {Q.p[k][0], Q.p[k][1], Q.p[k][2]};
      D3 q[3];
      for (int a = 0; a < 3; ++a) q[a] = dsum(dsum(dscale(p[0], R[a][0]), dscale(p[1], R[a][1])), dscale(p[2], R[a][2]));
      const D3 q2 = dsum(dsum(dmul(q[0], q[0]), dmul(q[1], q[1])), dmul(q[2], q[2]));
      const double* Sp = Q.S[k];
      D3 Sq[NS];
      solid_harmonics<L, D3, DualOps<double>>(q[0], q[1], q[2], q2, D3{1.0, 0.0, 0.0, 0.0}, Sq);
      const double w = Q.w[k];
      sh_for<L + 1>([&](auto IL) {
        constexpr int l = IL, n2 = 2 * l + 1, off = l * (2 * l - 1) * (2 * l + 1) / 3;
        const double wl = w * n2;
        sh_for<n2>([&](auto M) {
          const D3& sq = Sq[l * l + M];
          const double a = wl * (tx * sq.dx + ty * sq.dy + tz * sq.dz);
          sh_for<n2>([&](auto N) { acc[off + M * n2 + N] += a * Sp[l * l + N]; });
        });
      });
    }
  }
  for (int q = 0; q < ND; ++q) o[q] = T(acc[q]);
}

template <typename T, int L>
hipError_t wigner_jvp_T(int64_t n, const void* vec, const void* dvec, void* dD, hipStream_t s) {
  const int64_t blocks = (n + 63) / 64;
  hipLaunchKernelGGL((k_so2_wigner_jvp<T, L>), dim3((unsigned)blocks), dim3(64), 0, s, n,
                     static_cast<const T*>(vec), static_cast<const T*>(dvec), static_cast<T*>(dD));
  return hipGetLastError();
}

template <typename T>
hipError_t wigner_jvp_dispatch(int L, int64_t n, const void* vec, const void* dvec, void* dD, hipStream_t s) {
  switch (L) {
    case 0: return wigner_jvp_T<T, 0>(n, vec, dvec, dD, s);
    case 1: return wigner_jvp_T<T, 1>(n, vec, dvec, dD, s);
    case 2: return wigner_jvp_T<T, 2>(n, vec, dvec, dD, s);
    case 3: return wigner_jvp_T<T, 3>(n, vec, dvec, dD, s);
    case 4: return wigner_jvp_T<T, 4>(n, vec, dvec, dD, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int L>
hipError_t wigner_bwd_T(int64_t n, const void* vec, const void* gD, void* gvec, hipStream_t s) {
  const int64_t blocks = (n + 63) / 64;
  hipLaunchKernelGGL((k_so2_wigner_backward<T, L>), dim3((unsigned)blocks), dim3(64), 0, s, n,
                     static_cast<const T*>(vec), static_cast<const T*>(gD), static_cast<T*>(gvec));
  return hipGetLastError();
}

template <typename T>
hipError_t wigner_bwd_dispatch(int L, int64_t n, const void* vec, const void* gD, void* gvec, hipStream_t s) {
  switch (L) {
    case 0: return wigner_bwd_T<T, 0>(n, vec, gD, gvec, s);
    case 1: return wigner_bwd_T<T, 1>(n, vec, gD, gvec, s);
    case 2: return wigner_bwd_T<T, 2>(n, vec, gD, gvec, s);
    case 3: return wigner_bwd_T<T, 3>(n, vec, gD, gvec, s);
    case 4: return wigner_bwd_T<T, 4>(n, vec, gD, gvec, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int L>
hipError_t wigner_T(int64_t n, const void* vec, void* D, hipStream_t s) {
  const int64_t blocks = (n + 63) / 64;
  hipLaunchKernelGGL((k_so2_wigner<T, L>), dim3((unsigned)blocks), dim3(64), 0, s, n, static_cast<const T*>(vec),
                     static_cast<T*>(D));
  return hipGetLastError();
}

template <typename T>
hipError_t wigner_dispatch(int L, int64_t n, const void* vec, void* D, hipStream_t s) {
  switch (L) {
    case 0: return wigner_T<T, 0>(n, vec, D, s);
    case 1: return wigner_T<T, 1>(n, vec, D, s);
    case 2: return wigner_T<T, 2>(n, vec, D, s);
    case 3: return wigner_T<T, 3>(n, vec, D, s);
    case 4: return wigner_T<T, 4>(n, vec, D, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int L>
hipError_t sh_fwd_T(int64_t n, const void* vec, void* Y, hipStream_t s) {
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL((k_sh<T, L>), dim3((unsigned)blocks), dim3(256), 0, s, n, static_cast<const T*>(vec),
                     static_cast<T*>(Y));
  return hipGetLastError();
}
template <typename T, int L>
hipError_t sh_bwd_T(int64_t n, const void* vec, const void* gY, void* gvec, hipStream_t s) {
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL((k_sh_backward<T, L>), dim3((unsigned)blocks), dim3(256), 0, s, n, static_cast<const T*>(vec),
                     static_cast<const T*>(gY), static_cast<T*>(gvec));
  return hipGetLastError();
}

template <typename T>
hipError_t sh_dispatch(bool fwd, int L, int64_t n, const void* vec, const void* gY, void* out, hipStream_t s) {
  switch (L) {
    case 0: return fwd ? sh_fwd_T<T, 0>(n, vec, out, s) : sh_bwd_T<T, 0>(n, vec, gY, out, s);
    case 1: return fwd ? sh_fwd_T<T, 1>(n, vec, out, s) : sh_bwd_T<T, 1>(n, vec, gY, out, s);
    case 2: return fwd ? sh_fwd_T<T, 2>(n, vec, out, s) : sh_bwd_T<T, 2>(n, vec, gY, out, s);
    case 3: return fwd ? sh_fwd_T<T, 3>(n, vec, out, s) : sh_bwd_T<T, 3>(n, vec, gY, out, s);
    case 4: return fwd ? sh_fwd_T<T, 4>(n, vec, out, s) : sh_bwd_T<T, 4>(n, vec, gY, out, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_sh(int L, bool f64, int64_t n_edges, const void* vec, void* Y, hipStream_t s) {
  if (n_edges <= 0) return hipSuccess;
  return f64 ? sh_dispatch<double>(true, L, n_edges, vec, nullptr, Y, s)
             : sh_dispatch<float>(true, L, n_edges, vec, nullptr, Y, s);
}

hipError_t launch_sh_backward(int L, bool f64, int64_t n_edges, const void* vec, const void* grad_Y, void* grad_vec,
                              hipStream_t s) {
  if (n_edges <= 0) return hipSuccess;
  return f64 ? sh_dispatch<double>(false, L, n_edges, vec, grad_Y, grad_vec, s)
             : sh_dispatch<float>(false, L, n_edges, vec, grad_Y, grad_vec, s);
}

hipError_t launch_so2_wigner(int L, bool f64, int64_t n_edges, const void* vec, void* D, hipStream_t s) {
  if (n_edges <= 0) return hipSuccess;
  return f64 ? wigner_dispatch<double>(L, n_edges, vec, D, s) : wigner_dispatch<float>(L, n_edges, vec, D, s);
}

hipError_t launch_so2_wigner_backward(int L, bool f64, int64_t n_edges, const void* vec, const void* grad_D,
                                      void* grad_vec, hipStream_t s) {
  if (n_edges <= 0) return hipSuccess;
  return f64 ? wigner_bwd_dispatch<double>(L, n_edges, vec, grad_D, grad_vec, s)
             : wigner_bwd_dispatch<float>(L, n_edges, vec, grad_D, grad_vec, s);
}

hipError_t launch_so2_wigner_jvp(int L, bool f64, int64_t n_edges, const void* vec, const void* dvec, void* dD,
                                 hipStream_t s) {
  if (n_edges <= 0) return hipSuccess;
  return f64 ? wigner_jvp_dispatch<double>(L, n_edges, vec, dvec, dD, s)
             : wigner_jvp_dispatch<float>(L, n_edges, vec, dvec, dD, s);
}

hipError_t launch_pos_backward(bool f64, int64_t n_nodes, const int32_t* src_row, const int32_t* src_eid,
                               const int32_t* dst_row, const int32_t* dst_eid, const void* grad_vec, void* grad_pos,
                               hipStream_t s) {
  if (n_nodes <= 0) return hipSuccess;
  const int64_t blocks = (n_nodes + 3) / 4;
  if (f64)
    hipLaunchKernelGGL((k_pos_backward<double>), dim3((unsigned)blocks), dim3(256), 0, s, n_nodes, src_row, src_eid,
                       dst_row, dst_eid, static_cast<const double*>(grad_vec), static_cast<double*>(grad_pos));
  else
    hipLaunchKernelGGL((k_pos_backward<float>), dim3((unsigned)blocks), dim3(256), 0, s, n_nodes, src_row, src_eid,
                       dst_row, dst_eid, static_cast<const float*>(grad_vec), static_cast<float*>(grad_pos));
  return hipGetLastError();
}

}  // namespace tpconv
