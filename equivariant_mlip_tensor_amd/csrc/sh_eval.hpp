// sh_eval.hpp -- real spherical harmonics of an edge vector and their
// gradient, evaluated on the device in fp64.  Shared by the standalone
// harmonics kernels (sh.hip) and by the convolution kernels that evaluate the
// harmonics of each edge themselves (tp_kernels.hip), so both produce the
// same values.
//
// Harmonics: component-normalised real SH, Y_lm(r) = sqrt(2l+1) S_lm(r / |r|),
// with S_lm the real solid harmonics in Racah normalisation, built by their
// standard recurrences in l (sectoral terms from (x, y) and S_ll, S_l,-l; the
// rest from z S_lm and r^2 S_l-1,m).  This basis and sign convention equals
// the one of the real CG tables (real basis U^l over Condon-Shortley complex
// harmonics; Y_1 = sqrt(3) (y, z, x)).  A zero vector gets Y = (1, 0, ...)
// and a zero gradient.
#pragma once

#include <hip/hip_runtime.h>

#include <utility>

#include "cg_real.hpp"

namespace tpconv {
namespace shx {

template <typename F, int... I>
__device__ __forceinline__ void sh_sf(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void sh_for(F&& f) {
  if constexpr (N > 0) sh_sf(f, std::make_integer_sequence<int, N>{});
}

constexpr int lm_index(int l, int m) { return l * l + l + m; }

// recurrence coefficients (compile time)
constexpr double sect_coef(int l) {  // S_{l+1,+-(l+1)} from S_{l,+-l}
  return cg::csqrt((l == 0 ? 2.0 : 1.0) * (2 * l + 1) / (2.0 * l + 2.0));
}
constexpr double zc_coef(int l, int m) {  // (2l+1) / sqrt((l+m+1)(l-m+1))
  return (2.0 * l + 1.0) / cg::csqrt(double((l + m + 1) * (l - m + 1)));
}
constexpr double rc_coef(int l, int m) {  // sqrt((l+m)(l-m)) / sqrt((l+m+1)(l-m+1))
  return cg::csqrt(double((l + m) * (l - m))) / cg::csqrt(double((l + m + 1) * (l - m + 1)));
}

// A value and its gradient in (x, y, z): forward-mode derivatives through the
// recurrence, which treats x, y, z as free variables (r^2 = x^2 + y^2 + z^2),
// so each S_lm is the homogeneous polynomial and its gradient is exact.
template <typename T>
struct Dual {
  T v, dx, dy, dz;
};
template <typename T>
__device__ __forceinline__ Dual<T> dmul(const Dual<T>& a, const Dual<T>& b) {
  return {a.v * b.v, a.dx * b.v + a.v * b.dx, a.dy * b.v + a.v * b.dy, a.dz * b.v + a.v * b.dz};
}
template <typename T>
__device__ __forceinline__ Dual<T> dlin(T ca, const Dual<T>& a, T cb, const Dual<T>& b) {  // ca*a + cb*b
  return {ca * a.v + cb * b.v, ca * a.dx + cb * b.dx, ca * a.dy + cb * b.dy, ca * a.dz + cb * b.dz};
}
template <typename T>
__device__ __forceinline__ Dual<T> dscale(T c, const Dual<T>& a) {
  return {c * a.v, c * a.dx, c * a.dy, c * a.dz};
}

template <typename T>
struct PlainOps {
  static __device__ __forceinline__ T mul(T a, T b) { return a * b; }
  static __device__ __forceinline__ T lin(double ca, T a, double cb, T b) { return T(ca) * a + T(cb) * b; }
  static __device__ __forceinline__ T scale(double c, T a) { return T(c) * a; }
};
template <typename T>
struct DualOps {
  static __device__ __forceinline__ Dual<T> mul(const Dual<T>& a, const Dual<T>& b) { return dmul(a, b); }
  static __device__ __forceinline__ Dual<T> lin(double ca, const Dual<T>& a, double cb, const Dual<T>& b) {
    return dlin(T(ca), a, T(cb), b);
  }
  static __device__ __forceinline__ Dual<T> scale(double c, const Dual<T>& a) { return dscale(T(c), a); }
};

// S[lm] for l <= L at (x, y, z), r2 standing for x^2 + y^2 + z^2; N is T or
// Dual<T> and Ops supplies its product and linear combinations.
template <int L, typename N, class Ops>
__device__ __forceinline__ void solid_harmonics(const N& x, const N& y, const N& z, const N& r2, const N& one,
                                                N (&S)[(L + 1) * (L + 1)]) {
  S[0] = one;
  sh_for<L>([&](auto IL) {
    constexpr int l = IL;
    constexpr double c = sect_coef(l);
    if constexpr (l == 0) {
      S[lm_index(1, 1)] = x;
      S[lm_index(1, -1)] = y;
    } else {
      S[lm_index(l + 1, l + 1)] = Ops::lin(c, Ops::mul(x, S[lm_index(l, l)]), -c, Ops::mul(y, S[lm_index(l, -l)]));
      S[lm_index(l + 1, -(l + 1))] = Ops::lin(c, Ops::mul(y, S[lm_index(l, l)]), c, Ops::mul(x, S[lm_index(l, -l)]));
    }
    sh_for<2 * l + 1>([&](auto IM) {
      constexpr int m = int(IM) - l;
      constexpr double a = zc_coef(l, m);
      if constexpr (m >= -(l - 1) && m <= l - 1) {
        constexpr double b = rc_coef(l, m);
        S[lm_index(l + 1, m)] = Ops::lin(a, Ops::mul(z, S[lm_index(l, m)]), -b, Ops::mul(r2, S[lm_index(l - 1, m)]));
      } else {
        S[lm_index(l + 1, m)] = Ops::scale(a, Ops::mul(z, S[lm_index(l, m)]));
      }
    });
  });
}

template <typename T>
__device__ __forceinline__ double load_unit(const T* __restrict__ v, double& ux, double& uy, double& uz) {
  const double x = v[0], y = v[1], z = v[2];
  const double r = sqrt(x * x + y * y + z * z);
  const double inv = r > 0.0 ? 1.0 / r : 0.0;
  ux = x * inv;
  uy = y * inv;
  uz = z * inv;
  return r;
}

// Y_lm of the edge vector (vx, vy, vz) for l <= L, handed to put(k, value)
// with k = l*l + l + m, fp64 arithmetic.
template <int L, typename Put>
__device__ __forceinline__ void sh_values(double vx, double vy, double vz, Put&& put) {
  constexpr int D = (L + 1) * (L + 1);
  const double r = sqrt(vx * vx + vy * vy + vz * vz);
  const double inv = r > 0.0 ? 1.0 / r : 0.0;
  double S[D];
  solid_harmonics<L, double, PlainOps<double>>(vx * inv, vy * inv, vz * inv, 1.0, 1.0, S);
  const bool dir = r > 0.0;  // a zero vector keeps only Y_00 = 1
  sh_for<L + 1>([&](auto IL) {
    constexpr int l = IL;
    constexpr double nl = cg::csqrt(2.0 * l + 1.0);
    sh_for<2 * l + 1>([&](auto IM) {
      constexpr int k = l * l + int(IM);
      put(k, (dir || k == 0) ? nl * S[k] : 0.0);
    });
  });
}

// grad_vec = sum_lm g(k) dY_lm/dvec at (vx, vy, vz), k = l*l + l + m:
//   dY_lm/dvec = sqrt(2l+1) (grad S_lm(u) - l S_lm(u) u) / |r|,  u = r / |r|.
// sum_k w_k grad S_k(u) (w_k = sqrt(2l+1) g(k)) is the gradient of the
// polynomial F = sum_k w_k S_k, taken in reverse mode through the recurrence
// (x, y, z and r^2 as free variables, r^2 = 1 on the unit sphere): the values
// S and their adjoints A, 2 (L+1)^2 numbers in all.  Zero for a zero vector.
template <int L, typename Get>
__device__ __forceinline__ void sh_vec_grad(double vx, double vy, double vz, Get&& g, double& gx, double& gy,
                                            double& gz) {
  constexpr int D = (L + 1) * (L + 1);
  const double r = sqrt(vx * vx + vy * vy + vz * vz);
  if (!(r > 0.0)) {
    gx = gy = gz = 0.0;
    return;
  }
  const double inv = 1.0 / r;
  const double x = vx * inv, y = vy * inv, z = vz * inv;
  double S[D], A[D];
  solid_harmonics<L, double, PlainOps<double>>(x, y, z, 1.0, 1.0, S);
  double radial = 0.0;  // sum_k w_k l S_k
  sh_for<L + 1>([&](auto IL) {
    constexpr int l = IL;
    constexpr double nl = cg::csqrt(2.0 * l + 1.0);
    sh_for<2 * l + 1>([&](auto IM) {
      constexpr int k = l * l + int(IM);
      A[k] = nl * g(k);
      radial += double(l) * A[k] * S[k];
    });
  });
  double bx = 0.0, by = 0.0, bz = 0.0, br2 = 0.0;
  sh_for<L>([&](auto IR) {
    constexpr int l = L - 1 - int(IR);  // the step from level l to l + 1, last step first
    sh_for<2 * l + 1>([&](auto IM) {  // S[l+1, m] = a z S[l, m] - b r^2 S[l-1, m]
      constexpr int m = int(IM) - l;
      constexpr double ca = zc_coef(l, m);
      const double ab = A[lm_index(l + 1, m)];
      bz += ca * S[lm_index(l, m)] * ab;
      A[lm_index(l, m)] += ca * z * ab;
      if constexpr (m >= -(l - 1) && m <= l - 1) {
        constexpr double cb = rc_coef(l, m);
        br2 -= cb * S[lm_index(l - 1, m)] * ab;
        A[lm_index(l - 1, m)] -= cb * ab;
      }
    });
    if constexpr (l == 0) {  // S[1, 1] = x, S[1, -1] = y
      bx += A[lm_index(1, 1)];
      by += A[lm_index(1, -1)];
    } else {  // S[l+1, l+1] = c (x S_ll - y S_l,-l),  S[l+1, -l-1] = c (y S_ll + x S_l,-l)
      constexpr double c = sect_coef(l);
      const double pa = A[lm_index(l + 1, l + 1)], pb = A[lm_index(l + 1, -(l + 1))];
      const double sp = S[lm_index(l, l)], sm = S[lm_index(l, -l)];
      bx += c * (sp * pa + sm * pb);
      by += c * (sp * pb - sm * pa);
      A[lm_index(l, l)] += c * (x * pa + y * pb);
      A[lm_index(l, -l)] += c * (x * pb - y * pa);
    }
  });
  gx = (bx + 2.0 * x * br2 - radial * x) * inv;
  gy = (by + 2.0 * y * br2 - radial * y) * inv;
  gz = (bz + 2.0 * z * br2 - radial * z) * inv;
}

}  // namespace shx
}  // namespace tpconv
