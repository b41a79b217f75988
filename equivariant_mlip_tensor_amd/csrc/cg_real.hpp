// cg_real.hpp -- real-basis Clebsch-Gordan tables, usable at compile time.
//
// The tensor product runs over a sparse CG coefficient matrix stored as COO
// with its values deduplicated (FlashTP: Fused, Sparsity-Aware Tensor Product
// for Machine Learning Interatomic Potentials -- "Approach").  This header is
// the single builder of that matrix: the host plan (plan.cpp) calls it at run
// time to emit the COO table, and the kernels evaluate the same functions as
// constant expressions, so each nonzero becomes one FMA with a literal
// coefficient and compile-time register operands.
//
// Mathematics (textbook; the pages name the CG matrix but do not print it):
//  * complex CG <l1 m1 l2 m2 | l3 m3> by Racah's closed form, Condon-Shortley
//    phase.  The alternating sum times (l1+l2+l3)! is a sum of multinomial
//    coefficients, so it is evaluated exactly in int64; one sqrt and two
//    divisions in double follow.
//  * real basis: U^l, rows real m, columns complex mu,
//      m = 0 : U[0,0] = 1
//      m > 0 : U[m,m] = (-1)^m/sqrt2,  U[m,-m] = 1/sqrt2
//      m < 0 : U[m,m] = i/sqrt2,       U[m,-m] = -i(-1)^|m|/sqrt2
//    C_real[m1,m2,m3] = sum U1[m1,a] U2[m2,b] conj(U3[m3,c]) <l1 a l2 b|l3 c>,
//    real part for even l1+l2+l3, imaginary part for odd.
// Entries of a table are ordered by (m1, m2, m3); m indices are stored as
// m + l (0..2l).
#pragma once

#include <cstdint>

namespace tpconv {
namespace cg {

constexpr int kLMax = 4;                 // l bound of every table the kernels use
constexpr int kDimMax = 2 * kLMax + 1;
constexpr int kEntriesMax = kDimMax * kDimMax * kDimMax;

struct Entry {
  int8_t m1, m2, m3;   // m + l
  int8_t neg;          // coefficient sign
  double mag;          // |coefficient|
};

struct Table {
  int n = 0;
  Entry e[kEntriesMax] = {};
};

// n! for n <= 20 (exact in int64; exact in double as well)
struct FactTable {
  int64_t v[21] = {};
  constexpr FactTable() {
    v[0] = 1;
    for (int i = 1; i <= 20; ++i) v[i] = v[i - 1] * i;
  }
};
constexpr FactTable kFact{};

constexpr int64_t ifact(int n) { return kFact.v[n]; }

constexpr double dfact(int n) { return static_cast<double>(ifact(n)); }

// Newton iteration from above; converges to within one ulp of sqrt(a).
constexpr double csqrt(double a) {
  if (!(a > 0.0)) return 0.0;
  double x = a > 1.0 ? a : 1.0;
  for (int i = 0; i < 200; ++i) {
    const double nx = 0.5 * (x + a / x);
    if (nx >= x) break;
    x = nx;
  }
  return x;
}

constexpr bool triangle(int l1, int l2, int l3) {
  return (l1 - l2 <= l3 && l2 - l1 <= l3 && l3 <= l1 + l2);
}

constexpr int iabs(int v) { return v < 0 ? -v : v; }

// <l1 m1 l2 m2 | l3 m3>, Racah's formula.
constexpr double cg_complex(int l1, int m1, int l2, int m2, int l3, int m3) {
  if (m3 != m1 + m2 || !triangle(l1, l2, l3)) return 0.0;
  if (iabs(m1) > l1 || iabs(m2) > l2 || iabs(m3) > l3) return 0.0;
  const int n = l1 + l2 + l3;
  const int64_t nf = ifact(n);
  int64_t s = 0;  // (sum_k (-1)^k / prod of six factorials) * n!
  for (int k = 0; k <= n; ++k) {
    const int a[6] = {k, l1 + l2 - l3 - k, l1 - m1 - k, l2 + m2 - k, l3 - l2 + m1 + k, l3 - l1 - m2 + k};
    bool ok = true;
    int64_t den = 1;
    for (int t = 0; t < 6; ++t) {
      if (a[t] < 0) ok = false;
    }
    if (!ok) continue;
    for (int t = 0; t < 6; ++t) den *= ifact(a[t]);
    s += ((k & 1) ? -1 : 1) * (nf / den);  // six arguments sum to n: a multinomial coefficient
  }
  if (s == 0) return 0.0;
  const double num = (2.0 * l3 + 1.0) * dfact(l3 + l1 - l2) * dfact(l3 - l1 + l2) * dfact(l1 + l2 - l3) *
                     dfact(l3 + m3) * dfact(l3 - m3) * dfact(l1 - m1) * dfact(l1 + m1) * dfact(l2 - m2) *
                     dfact(l2 + m2);
  return static_cast<double>(s) / dfact(n) * csqrt(num / dfact(n + 1));
}

struct Cplx {
  double re = 0.0, im = 0.0;
};

constexpr Cplx cmul(Cplx a, Cplx b) { return {a.re * b.re - a.im * b.im, a.re * b.im + a.im * b.re}; }

// Nonzeros of row m of U^l: up to two (mu, coefficient) pairs.
struct URow {
  int n = 0;
  int mu[2] = {0, 0};
  Cplx c[2] = {};
};

constexpr URow urow(int m) {
  URow r;
  const double h = csqrt(0.5);
  if (m == 0) {
    r.n = 1;
    r.mu[0] = 0;
    r.c[0] = {1.0, 0.0};
  } else if (m > 0) {
    r.n = 2;
    r.mu[0] = m;
    r.c[0] = {(m & 1) ? -h : h, 0.0};
    r.mu[1] = -m;
    r.c[1] = {h, 0.0};
  } else {
    const int k = -m;
    r.n = 2;
    r.mu[0] = -k;
    r.c[0] = {0.0, h};
    r.mu[1] = k;
    r.c[1] = {0.0, (k & 1) ? h : -h};  // -i (-1)^k / sqrt2
  }
  return r;
}

// Real-basis coefficient C[m1, m2, m3] (m in -l..l).
constexpr double cg_real_value(int l1, int m1, int l2, int m2, int l3, int m3) {
  // only |m3| = |m1| + |m2| or ||m1| - |m2|| can couple
  const int a1 = iabs(m1), a2 = iabs(m2), a3 = iabs(m3);
  if (a3 != a1 + a2 && a3 != iabs(a1 - a2)) return 0.0;
  const URow r1 = urow(m1), r2 = urow(m2), r3 = urow(m3);
  Cplx acc;
  for (int i = 0; i < r1.n; ++i)
    for (int j = 0; j < r2.n; ++j)
      for (int k = 0; k < r3.n; ++k) {
        if (r3.mu[k] != r1.mu[i] + r2.mu[j]) continue;
        const double c = cg_complex(l1, r1.mu[i], l2, r2.mu[j], l3, r3.mu[k]);
        if (c == 0.0) continue;
        const Cplx conj3 = {r3.c[k].re, -r3.c[k].im};
        const Cplx t = cmul(cmul(r1.c[i], r2.c[j]), conj3);
        acc.re += t.re * c;
        acc.im += t.im * c;
      }
  const double v = ((l1 + l2 + l3) % 2 == 0) ? acc.re : acc.im;
  return (v < 1e-12 && v > -1e-12) ? 0.0 : v;
}

constexpr Table build_table(int l1, int l2, int l3) {
  Table t;
  if (!triangle(l1, l2, l3) || l1 > kLMax || l2 > kLMax || l3 > kLMax || l1 < 0 || l2 < 0 || l3 < 0) return t;
  for (int m1 = -l1; m1 <= l1; ++m1)
    for (int m2 = -l2; m2 <= l2; ++m2)
      for (int m3 = -l3; m3 <= l3; ++m3) {
        const double v = cg_real_value(l1, m1, l2, m2, l3, m3);
        if (v == 0.0) continue;
        Entry& e = t.e[t.n++];
        e.m1 = static_cast<int8_t>(m1 + l1);
        e.m2 = static_cast<int8_t>(m2 + l2);
        e.m3 = static_cast<int8_t>(m3 + l3);
        e.neg = v < 0.0 ? 1 : 0;
        e.mag = v < 0.0 ? -v : v;
      }
  return t;
}

// Compile-time access: one constant table per (l1, l2, l3).
template <int L1, int L2, int L3>
struct TableOf {
  static constexpr Table value = build_table(L1, L2, L3);
};

}  // namespace cg
}  // namespace tpconv
