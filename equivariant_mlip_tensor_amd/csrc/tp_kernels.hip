// tp_kernels.hip -- fused CGTP convolution kernels for gfx950 (CDNA4).
//
// Compiled once per l bound, data type and kernel family (-DTPCONV_L=0..4,
// -DTPCONV_DOUBLE=0|1, -DTPCONV_DD=0|1); each object defines that triple's two launchers
// declared in tp_common.hpp.
//
// Execution (node-centric, LunaTP Abstract; one fused kernel per direction,
// FlashTP "Approach"):
//  * one 64-lane wavefront per CSR row (destination node in the forward,
//    source node in the backward);
//  * lanes = edge slot x channel: a slot is a power-of-two group of lanes
//    >= U, so a wave walks 64/slot edges of its row side by side;
//  * each lane gathers its channel of the neighbour's irreps, the edge's SH
//    row and its channel of every path weight, and keeps all per-node
//    accumulators in registers for the whole row -- no per-edge tensor is
//    written in the forward, and the row's sum is formed in registers and
//    across slots with lane shuffles, never with global atomics;
//  * the CG table is unrolled at compile time from cg_real.hpp: every
//    nonzero is one FMA with a literal coefficient and register operands;
//    products x[m1]*Y[m2] are formed once per (l1, l2) group and shared by
//    all paths of the group (path aggregation, FlashTP "Approach" and its
//    measured-effects table).
//
// Two plan policies instantiate the same code: FullPlan<L, U> for plans whose
// segments are l = 0..L in order with natural parity (every offset, path and
// lane mapping a compile-time constant, no branch inside an edge), and
// RtPlan<L, PAR> for any other plan (path set, offsets and U read from the
// launch arguments, one uniform branch per path).
//
// With TPCONV_DD=1 the same two row kernels compute the double backward
// (FwdDD: grad_G over destination rows; BwdDD: grad_x, grad_Y, grad_W over
// source rows).  Beyond the scheme above:
//  * the fp32 backward issues the next edge's loads before this edge's
//    stores, into a second register set (bwd_pipelined);
//  * graphs with at most 1024 rows split each row over the 4 waves of a
//    block, which meet in LDS (row_part, template parameter R);
//  * fp64 contractions sum the products that share an (m3, |c|) pair before
//    one multiply by the coefficient (Grouped), because an fp64 coefficient
//    is no inline literal; the fp64 forward and double-backward grad_G pass
//    form each product where it is summed (an FMA per entry) instead of once
//    per (l1, l2) group.
//
// With KernelArgs::from_vec set (template parameter YS = kYVec; one launch per plan) the forward and
// backward evaluate each edge's harmonics themselves from the edge vector
// (sh_eval.hpp, fp64, one lane per edge for a chunk of the row's edges at a
// time, kept in a per-wave LDS block the slots read), and the backward turns
// each chunk's channel-summed dY, kept in LDS, into grad_vec [E][3] the same
// way: Y and dY never reach device memory.
#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>

#include "sh_eval.hpp"
#include "tp_common.hpp"

#ifndef TPCONV_L
#error "compile with -DTPCONV_L=<l bound>"
#endif
#ifndef TPCONV_DOUBLE
#error "compile with -DTPCONV_DOUBLE=0 (fp32) or 1 (fp64)"
#endif
#ifndef TPCONV_DD
#error "compile with -DTPCONV_DD=0 (forward, backward) or 1 (double backward)"
#endif

namespace tpconv {
namespace {

template <typename F, int... I>
__device__ __forceinline__ void sf_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) sf_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ float fmaT(float a, float b, float c) { return __builtin_fmaf(a, b, c); }
__device__ __forceinline__ double fmaT(double a, double b, double c) { return __builtin_fma(a, b, c); }

// Empty asm that keeps a value in a VGPR as an opaque SSA value.
template <typename T>
__device__ __forceinline__ void pin_vgpr(T& v) {
  asm volatile("" : "+v"(v));
}

template <typename T>
__device__ __forceinline__ T ldg_stream(const T* p) {
  return __builtin_nontemporal_load(p);
}

// Orders one wavefront's LDS accesses around a hand-over between its lanes
// (one lane writes, another reads): a code-motion barrier for the compiler;
// the hardware runs a wavefront's LDS instructions in order.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Where a kernel takes each edge's harmonics from (template parameter YS):
// every lane of the edge's slot loads the row from Y (kYGlobal); one lane per
// edge evaluates them from the edge vector into the wave's LDS block for a
// chunk of the row's edges (kYVec); or, in the forward, one lane per edge
// copies the Y row into that block (kYRows: c4k forward 0.150 -> 0.147 ms;
// the same staging of Y and dY rows made the backward slower, 0.316 ->
// 0.330 ms, so the backward loads per slot).
constexpr int kYGlobal = 0, kYVec = 1, kYRows = 2;

// Row accumulators: a row sums one term per edge, so for fp32 data it is
// kept in fp64 (full rate on CDNA); each edge's own sum over its paths stays
// in the data type.
template <typename T>
struct RowAcc {
  using type = T;
};
template <>
struct RowAcc<float> {
  using type = double;
};

enum Parity { kAnyParity = 0, kEvenOnly = 1 };


constexpr bool triple_in_class(int l1, int l2, int l3, int par) {
  return par == kAnyParity || ((l1 + l2 + l3) % 2 == 0);
}

constexpr int log2_ceil(int n) {
  int k = 0;
  while ((1 << k) < n) ++k;
  return k;
}

// ----------------------------------------------------- triple bookkeeping
struct TripleInfo {
  int l1 = -1, l2 = -1, l3 = -1;
};

constexpr TripleInfo triple_at(int L, int t) {
  int n = 0;
  for (int a = 0; a <= L; ++a)
    for (int b = 0; b <= L; ++b)
      for (int c = 0; c <= L; ++c)
        if (cg::triangle(a, b, c)) {
          if (n == t) return TripleInfo{a, b, c};
          ++n;
        }
  return TripleInfo{};
}

constexpr bool triple_even(int L, int t) {
  const TripleInfo i = triple_at(L, t);
  return ((i.l1 + i.l2 + i.l3) % 2) == 0;
}

// rank of triple t among the even triples (its path index in a full plan)
constexpr int even_rank(int L, int t) {
  int r = 0;
  for (int s = 0; s < t; ++s)
    if (triple_even(L, s)) ++r;
  return r;
}

constexpr int even_count(int L) { return even_rank(L, triple_count(L)); }

constexpr bool even_first3(int L, int t) {
  const int l3 = triple_at(L, t).l3;
  for (int s = 0; s < t; ++s)
    if (triple_even(L, s) && triple_at(L, s).l3 == l3) return false;
  return true;
}

// Backward visits paths in (l3, l1, l2) order, so the products |c| * G[m3]
// shared by paths into the same l3 stay inside one block of code.
constexpr int bwd_pos(int L, int l1, int l2, int l3) { return (l3 * (L + 1) + l1) * (L + 1) + l2; }

constexpr bool even_first1_bwd(int L, int t) {
  const TripleInfo me = triple_at(L, t);
  const int pos = bwd_pos(L, me.l1, me.l2, me.l3);
  for (int s = 0; s < triple_count(L); ++s) {
    const TripleInfo o = triple_at(L, s);
    if (triple_even(L, s) && o.l1 == me.l1 && bwd_pos(L, o.l1, o.l2, o.l3) < pos) return false;
  }
  return true;
}

__device__ __forceinline__ bool bit(uint64_t lo, uint64_t hi, int t) {
  return t < 64 ? ((lo >> t) & 1ull) : ((hi >> (t - 64)) & 1ull);
}

// ------------------------------------------------------------- policies
template <int L, int PAR>
struct RtPlan {
  static constexpr int kPar = PAR;
  static constexpr bool kFull = false;
  static __device__ __forceinline__ int lps_log2(const KernelArgs& a) { return a.lps_log2; }
  static __device__ __forceinline__ int nslots(const KernelArgs& a) { return a.nslots; }
  static __device__ __forceinline__ int mul(const KernelArgs& a) { return a.mul; }
  static __device__ __forceinline__ int d_in(const KernelArgs& a) { return a.d_in; }
  static __device__ __forceinline__ int d_out(const KernelArgs& a) { return a.d_out; }
  static __device__ __forceinline__ int d_sh(const KernelArgs& a) { return a.d_sh; }
  static __device__ __forceinline__ int64_t wstride(const KernelArgs& a) { return a.wstride; }
  static __device__ __forceinline__ int in_off(const KernelArgs& a, int l) { return a.in_off[l]; }
  static __device__ __forceinline__ int out_off(const KernelArgs& a, int l) { return a.out_off[l]; }
  static __device__ __forceinline__ bool in_l(const KernelArgs& a, int l) { return (a.in_l_mask >> l) & 1; }
  static __device__ __forceinline__ bool out_l(const KernelArgs& a, int l) { return (a.out_l_mask >> l) & 1; }
  template <int t>
  static __device__ __forceinline__ bool on(const KernelArgs& a) {
    return bit(a.pmask_lo, a.pmask_hi, t);
  }
  template <int t>
  static __device__ __forceinline__ bool first3(const KernelArgs& a) {
    return bit(a.first3_lo, a.first3_hi, t);
  }
  template <int t>
  static __device__ __forceinline__ bool first1(const KernelArgs& a) {
    return bit(a.first1_lo, a.first1_hi, t);
  }
  template <int t>
  static __device__ __forceinline__ int woff(const KernelArgs& a) {
    return a.woff[t];
  }
  // guard of a path's arithmetic
  template <int t>
  static __device__ __forceinline__ bool run(const KernelArgs& a, int) {
    return on<t>(a);
  }
};

template <int L, int U>
struct FullPlan {
  static_assert(U >= 1 && U <= 64, "one wave holds at most 64 channels");
  static constexpr int kPar = kEvenOnly;
  static constexpr bool kFull = true;
  static constexpr int kLg = log2_ceil(U);
  static constexpr int kD = U * (L + 1) * (L + 1);
  static __device__ __forceinline__ constexpr int lps_log2(const KernelArgs&) { return kLg; }
  static __device__ __forceinline__ constexpr int nslots(const KernelArgs&) { return 64 >> kLg; }
  static __device__ __forceinline__ constexpr int mul(const KernelArgs&) { return U; }
  static __device__ __forceinline__ constexpr int d_in(const KernelArgs&) { return kD; }
  static __device__ __forceinline__ constexpr int d_out(const KernelArgs&) { return kD; }
  static __device__ __forceinline__ constexpr int d_sh(const KernelArgs&) { return (L + 1) * (L + 1); }
  static __device__ __forceinline__ constexpr int64_t wstride(const KernelArgs&) {
    constexpr int64_t v = int64_t(U) * even_count(L);
    return v;
  }
  static __device__ __forceinline__ constexpr int in_off(const KernelArgs&, int l) { return U * l * l; }
  static __device__ __forceinline__ constexpr int out_off(const KernelArgs&, int l) { return U * l * l; }
  static __device__ __forceinline__ constexpr bool in_l(const KernelArgs&, int) { return true; }
  static __device__ __forceinline__ constexpr bool out_l(const KernelArgs&, int) { return true; }
  // constexpr locals force compile-time evaluation of the helpers
  template <int t>
  static __device__ __forceinline__ constexpr bool on(const KernelArgs&) {
    constexpr bool v = triple_even(L, t);
    return v;
  }
  template <int t>
  static __device__ __forceinline__ constexpr bool first3(const KernelArgs&) {
    constexpr bool v = even_first3(L, t);
    return v;
  }
  template <int t>
  static __device__ __forceinline__ constexpr bool first1(const KernelArgs&) {
    constexpr bool v = even_first1_bwd(L, t);
    return v;
  }
  template <int t>
  static __device__ __forceinline__ constexpr int woff(const KernelArgs&) {
    constexpr int v = even_rank(L, t) * U;
    return v;
  }
  // Guard of a path's arithmetic: `tok` is the wave's first edge id of this
  // iteration, never negative, but unknown to the compiler, different in
  // every iteration and copied through a scalar move per path, so every path
  // stays its own basic block.  Without these block boundaries the compiler
  // schedules the whole edge as one block, hoists products across paths and
  // runs out of registers.
  template <int t>
  static __device__ __forceinline__ bool run(const KernelArgs&, int tok) {
    int v;
    asm volatile("s_mov_b32 %0, %1" : "=s"(v) : "s"(tok));  // opaque per path: no merging of guards
    return v >= 0;
  }
};

// A full plan restricted to the paths into the output l's in OUT (bit l):
// the forward of a plan too wide for the register file runs as launches over
// disjoint sets of output l's, each writing only its own output columns.
template <int L, int U, int OUT>
struct FullPlanPart : FullPlan<L, U> {
  template <int t>
  static __device__ __forceinline__ constexpr bool on(const KernelArgs&) {
    constexpr bool v = triple_even(L, t) && ((OUT >> triple_at(L, t).l3) & 1);
    return v;
  }
  static __device__ __forceinline__ constexpr int out_off(const KernelArgs&, int l) {
    return ((OUT >> l) & 1) ? U * l * l : -1;
  }
  static __device__ __forceinline__ constexpr bool out_l(const KernelArgs&, int l) { return (OUT >> l) & 1; }
};

// Compile-time facts about a CG table.
template <int L1, int L2, int L3>
struct TabInfo {
  static constexpr const cg::Table& tab = cg::TableOf<L1, L2, L3>::value;
  static constexpr bool first_m3(int k) {
    for (int j = 0; j < k; ++j)
      if (tab.e[j].m3 == tab.e[k].m3) return false;
    return true;
  }
  static constexpr bool first_m1(int k) {
    for (int j = 0; j < k; ++j)
      if (tab.e[j].m1 == tab.e[k].m1) return false;
    return true;
  }
  static constexpr bool first_m2(int k) {
    for (int j = 0; j < k; ++j)
      if (tab.e[j].m2 == tab.e[k].m2) return false;
    return true;
  }
  static constexpr bool has_m1(int m) {
    for (int j = 0; j < tab.n; ++j)
      if (tab.e[j].m1 == m) return true;
    return false;
  }
  static constexpr bool has_m2(int m) {
    for (int j = 0; j < tab.n; ++j)
      if (tab.e[j].m2 == m) return true;
    return false;
  }
  static constexpr bool has_m3(int m) {
    for (int j = 0; j < tab.n; ++j)
      if (tab.e[j].m3 == m) return true;
    return false;
  }
  // A path with an l = 0 leg couples by one coefficient c for every m:
  // (l, 0, l) as c x[m] Y0, (0, l, l) as c x0 Y[m] (the identity, c = 1), and
  // (l, l, 0) as c times the dot product x . Y.  kDiag: 1, 2, 3 for these
  // forms, 0 for any other path (or a table not of that form).  The table's
  // fp64 values carry the builder's rounding (0.99999999999999978 for 1), so
  // magnitudes are compared to 1e-14 relative, and the identity uses c = 1.
  static constexpr bool near(double a, double b) {
    const double d = a > b ? a - b : b - a;
    return d <= 1e-14 * (a > 0 ? a : -a);
  }
  static constexpr int diag_kind() {
    const int kind = L2 == 0 ? 1 : L1 == 0 ? 2 : L3 == 0 ? 3 : 0;
    if (kind == 0) return 0;
    const int l = kind == 2 ? L2 : L1;
    if (tab.n != 2 * l + 1) return 0;
    if (kind != 3 && (tab.e[0].neg || !near(tab.e[0].mag, 1.0))) return 0;
    bool seen[2 * cg::kLMax + 1] = {};
    for (int j = 0; j < tab.n; ++j) {
      const cg::Entry& en = tab.e[j];
      if (!near(en.mag, tab.e[0].mag) || en.neg != tab.e[0].neg) return 0;
      int m = en.m1;
      if (kind == 1 && (en.m2 != 0 || en.m1 != en.m3)) return 0;
      if (kind == 2 && (en.m1 != 0 || en.m2 != en.m3)) return 0;
      if (kind == 3 && (en.m3 != 0 || en.m1 != en.m2)) return 0;
      if (kind == 2) m = en.m2;
      if (seen[m]) return 0;
      seen[m] = true;
    }
    return kind;
  }
  static constexpr int kDiag = diag_kind();
  static constexpr double kDiagCoef = kDiag == 1 || kDiag == 2 ? 1.0 : tab.e[0].neg ? -tab.e[0].mag : tab.e[0].mag;
};

// The table's entries grouped by (m3, |c|), for fp64 kernels: an fp64
// coefficient is no inline literal, so every use costs two scalar moves; in
// z[m3] += c (+-p1 +- p2 ...) each distinct coefficient is used once per
// group.  Inside a group a positive entry comes first (no negation needed);
// a group with only negative entries sums magnitudes and uses -c.
template <int L1, int L2, int L3>
struct Grouped {
  static constexpr const cg::Table& tab = cg::TableOf<L1, L2, L3>::value;
  struct Order {
    int n = 0;
    int idx[cg::kEntriesMax] = {};      // entry at this position
    bool open[cg::kEntriesMax] = {};    // first of its group
    bool close[cg::kEntriesMax] = {};   // last of its group
    bool first_m3[cg::kEntriesMax] = {};// the group is the first one of its m3
    bool flip[cg::kEntriesMax] = {};    // group of negative entries only (at close)
    bool sub[cg::kEntriesMax] = {};     // subtract this entry (not at open)
  };
  static constexpr Order build() {
    Order o;
    bool used[cg::kEntriesMax] = {};
    bool seen_m3[2 * cg::kLMax + 1] = {};
    for (int a = 0; a < tab.n; ++a) {
      if (used[a]) continue;
      // members of a's group, positive ones first
      int mem[cg::kEntriesMax] = {};
      int k = 0;
      for (int pass = 0; pass < 2; ++pass)
        for (int b = a; b < tab.n; ++b)
          if (!used[b] && tab.e[b].m3 == tab.e[a].m3 && tab.e[b].mag == tab.e[a].mag &&
              (tab.e[b].neg != 0) == (pass == 1))
            mem[k++] = b;
      const bool all_neg = tab.e[mem[0]].neg != 0;
      for (int j = 0; j < k; ++j) {
        const int pos = o.n++;
        used[mem[j]] = true;
        o.idx[pos] = mem[j];
        o.open[pos] = j == 0;
        o.close[pos] = j == k - 1;
        o.sub[pos] = j > 0 && !all_neg && tab.e[mem[j]].neg != 0;
        o.flip[pos] = all_neg;
        o.first_m3[pos] = !seen_m3[tab.e[mem[j]].m3];
      }
      seen_m3[tab.e[a].m3] = true;
    }
    return o;
  }
  static constexpr Order ord = build();
};

// Is product x[m1]*Y[m2] used by some table of group (l1, l2) in parity class PAR?
template <int L, int PAR, int L1, int L2, int L3 = 0>
constexpr bool group_uses(int m1, int m2) {
  if constexpr (L3 > L) {
    return false;
  } else {
    bool used = false;
    if constexpr (cg::triangle(L1, L2, L3) && triple_in_class(L1, L2, L3, PAR)) {
      const cg::Table& t = cg::TableOf<L1, L2, L3>::value;
      for (int j = 0; j < t.n; ++j)
        if (t.e[j].m1 == m1 && t.e[j].m2 == m2) used = true;
    }
    return used || group_uses<L, PAR, L1, L2, L3 + 1>(m1, m2);
  }
}

template <int L, class P, int L1, int L2>
__device__ __forceinline__ bool group_on(const KernelArgs& a) {
  bool any = false;
  static_for<L + 1>([&](auto I3) {
    constexpr int l3 = I3;
    if constexpr (cg::triangle(L1, L2, l3) && triple_in_class(L1, L2, l3, P::kPar))
      any = any || P::template on<triple_id(L, L1, L2, l3)>(a);
  });
  return any;
}

// w[t] = this lane's channel of path t in weight row e
template <typename T, int L, class P>
__device__ __forceinline__ void load_w(const KernelArgs& a, const T* __restrict__ Wp, int64_t wstride, int uc, int e,
                                       T (&w)[triple_count(L)]) {
  const T* wr = Wp + (int64_t)e * wstride + uc;
  static_for<triple_count(L)>([&](auto I) {
    constexpr TripleInfo ti = triple_at(L, I);
    if constexpr (triple_in_class(ti.l1, ti.l2, ti.l3, P::kPar)) {
      if (P::template on<I>(a)) w[I] = ldg_stream(wr + P::template woff<I>(a));
      else w[I] = T(0);
    } else {
      w[I] = T(0);
    }
  });
}

// The double backward's grad_G kernel for l = 4 holds more per-edge state
// than the register file (it spills to scratch): it keeps the row sum in an
// LDS slab for fp64 data too.  (For the plain forward the per-edge slab
// update costs more than the registers it frees.)
template <typename T, int L, bool DD>
constexpr bool row_sum_in_lds() {
  return DD && L >= 4;
}

// ------------------------------------------------------------------ forward
template <typename T, int L, class P>
struct Fwd {
  static constexpr int NL = (L + 1) * (L + 1);
  static constexpr int NT = triple_count(L);

  // te[l3 block] = sum over the edge's paths into l3 of W[p,u] * CG_p(x, y)
  static __device__ __forceinline__ void edge(const KernelArgs& a, int tok, const T (&x)[NL], const T (&y)[NL],
                                              const T (&w)[NT], T (&te)[NL]) {
    static_for<L + 1>([&](auto I1) {
      constexpr int l1 = I1;
      static_for<L + 1>([&](auto I2) {
        constexpr int l2 = I2;
        if (!group_on<L, P, l1, l2>(a)) return;
        constexpr int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1;
        // a group with an l = 0 leg holds the one path (l1, l2, max(l1, l2));
        // its weight and scalar factor are folded first, so no products
        constexpr bool kDiagGroup = (l1 == 0 || l2 == 0) && TabInfo<l1, l2, (l1 > l2 ? l1 : l2)>::kDiag != 0;
        // fp64: each product x[m1] Y[m2] is formed where its entry is summed
        // (one FMA per entry in place of a product per pair plus an add per
        // entry): fewer instructions and no product array in registers
        constexpr bool kAtUse = sizeof(T) == 8;
        T pr[n1 * n2];
        static_for<n1>([&](auto M1) {
          static_for<n2>([&](auto M2) {
            if constexpr (!kAtUse && !kDiagGroup && group_uses<L, P::kPar, l1, l2>(M1, M2))
              pr[M1 * n2 + M2] = x[l1 * l1 + M1] * y[l2 * l2 + M2];
          });
        });
        static_for<L + 1>([&](auto I3) {
          constexpr int l3 = I3;
          if constexpr (cg::triangle(l1, l2, l3) && triple_in_class(l1, l2, l3, P::kPar)) {
            constexpr int t = triple_id(L, l1, l2, l3);
            if (P::template on<t>(a) && P::template run<t>(a, tok)) {
              using TI = TabInfo<l1, l2, l3>;
              constexpr int n3 = 2 * l3 + 1;
              if constexpr (kDiagGroup) {
                // (l, 0, l): te += (W c Y0) x;  (0, l, l): te += (W c x0) Y
                static_assert(TI::kDiag == 1 || TI::kDiag == 2, "l = 0 leg without the identity form");
                constexpr T c = T(TI::kDiagCoef);
                const T f = w[t] * (TI::kDiag == 1 ? c * y[0] : c * x[0]);
                static_for<n3>([&](auto M3) {
                  const T v = TI::kDiag == 1 ? x[l1 * l1 + M3] : y[l2 * l2 + M3];
                  if (P::template first3<t>(a)) te[l3 * l3 + M3] = f * v;
                  else te[l3 * l3 + M3] = fmaT(f, v, te[l3 * l3 + M3]);
                });
              } else {
                T z[n3];
                if constexpr (sizeof(T) == 8) {
                  using GR = Grouped<l1, l2, l3>;
                  T acc_g = T(0);
                  static_for<GR::ord.n>([&](auto K) {
                    constexpr cg::Entry en = TI::tab.e[GR::ord.idx[K]];
                    if constexpr (kAtUse) {
                      const T xv = x[l1 * l1 + en.m1], yv = y[l2 * l2 + en.m2];
                      if constexpr (GR::ord.open[K]) acc_g = xv * yv;
                      else if constexpr (GR::ord.sub[K]) acc_g = fmaT(-xv, yv, acc_g);
                      else acc_g = fmaT(xv, yv, acc_g);
                    } else {
                      const T p = pr[en.m1 * n2 + en.m2];
                      if constexpr (GR::ord.open[K]) acc_g = p;
                      else if constexpr (GR::ord.sub[K]) acc_g = acc_g - p;
                      else acc_g = acc_g + p;
                    }
                    if constexpr (GR::ord.close[K]) {
                      constexpr T c = GR::ord.flip[K] ? T(-en.mag) : T(en.mag);
                      if constexpr (GR::ord.first_m3[K])
                        z[en.m3] = c * acc_g;
                      else
                        z[en.m3] = fmaT(c, acc_g, z[en.m3]);
                    }
                  });
                } else {
                  static_for<TI::tab.n>([&](auto K) {
                    constexpr cg::Entry en = TI::tab.e[K];
                    constexpr T c = en.neg ? T(-en.mag) : T(en.mag);
                    const T p = pr[en.m1 * n2 + en.m2];
                    if constexpr (TI::first_m3(K))
                      z[en.m3] = c * p;
                    else
                      z[en.m3] = fmaT(c, p, z[en.m3]);
                  });
                }
                if (P::template first3<t>(a)) {
                  static_for<n3>([&](auto M3) { te[l3 * l3 + M3] = w[t] * z[M3]; });
                } else {
                  static_for<n3>([&](auto M3) { te[l3 * l3 + M3] = fmaT(w[t], z[M3], te[l3 * l3 + M3]); });
                }
              }
            }
          }
        });
      });
    });
  }
};

// Double backward, grad_G: with a, b, c the cotangents of grad_x, grad_Y and
// grad_W, te[l3 block] = sum over the edge's paths of
//   W[p,u] * CG_p(a, y) + W[p,u] * CG_p(x, b) + c[p,u] * CG_p(x, y).
// The first two share one product array per group, p2 = a (x) y + x (x) b.
template <typename T, int L, class P>
struct FwdDD {
  static constexpr int NL = (L + 1) * (L + 1);
  static constexpr int NT = triple_count(L);

  static __device__ __forceinline__ void edge(const KernelArgs& a, int tok, const T (&x)[NL], const T (&xa)[NL],
                                              const T (&y)[NL], const T (&yb)[NL], const T (&w)[NT],
                                              const T (&wc)[NT], T (&te)[NL]) {
    static_for<L + 1>([&](auto I1) {
      constexpr int l1 = I1;
      static_for<L + 1>([&](auto I2) {
        constexpr int l2 = I2;
        if (!group_on<L, P, l1, l2>(a)) return;
        constexpr int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1;
        constexpr bool kDiagGroup = (l1 == 0 || l2 == 0) && TabInfo<l1, l2, (l1 > l2 ? l1 : l2)>::kDiag != 0;
        // fp64: products formed where each entry is summed, as in the forward
        constexpr bool kAtUse = sizeof(T) == 8;
        T p1[n1 * n2], p2[n1 * n2];
        static_for<n1>([&](auto M1) {
          static_for<n2>([&](auto M2) {
            if constexpr (!kAtUse && !kDiagGroup && group_uses<L, P::kPar, l1, l2>(M1, M2)) {
              const T xv = x[l1 * l1 + M1], yv = y[l2 * l2 + M2];
              p1[M1 * n2 + M2] = xv * yv;
              p2[M1 * n2 + M2] = fmaT(xa[l1 * l1 + M1], yv, xv * yb[l2 * l2 + M2]);
            }
          });
        });
        static_for<L + 1>([&](auto I3) {
          constexpr int l3 = I3;
          if constexpr (cg::triangle(l1, l2, l3) && triple_in_class(l1, l2, l3, P::kPar)) {
            constexpr int t = triple_id(L, l1, l2, l3);
            if (P::template on<t>(a) && P::template run<t>(a, tok)) {
              using TI = TabInfo<l1, l2, l3>;
              constexpr int n3 = 2 * l3 + 1;
              if constexpr (kDiagGroup) {
                // with k the path's coefficient and c the weight cotangent:
                // (l, 0, l): te += (W k Y0) a + (W k b0 + c k Y0) x
                // (0, l, l): te += (W k x0) b + (W k a0 + c k x0) Y
                static_assert(TI::kDiag == 1 || TI::kDiag == 2, "l = 0 leg without the identity form");
                constexpr T c = T(TI::kDiagCoef);
                constexpr bool k1 = TI::kDiag == 1;
                const T sm = c * (k1 ? y[0] : x[0]);
                const T so = c * (k1 ? yb[0] : xa[0]);
                const T f1 = w[t] * sm;
                const T f2 = fmaT(w[t], so, wc[t] * sm);
                static_for<n3>([&](auto M3) {
                  const T v1 = k1 ? xa[l1 * l1 + M3] : yb[l2 * l2 + M3];
                  const T v2 = k1 ? x[l1 * l1 + M3] : y[l2 * l2 + M3];
                  if (P::template first3<t>(a)) te[l3 * l3 + M3] = fmaT(f1, v1, f2 * v2);
                  else te[l3 * l3 + M3] = fmaT(f1, v1, fmaT(f2, v2, te[l3 * l3 + M3]));
                });
                return;
              }
              T z1[n3], z2[n3];
              if constexpr (sizeof(T) == 8) {
                using GR = Grouped<l1, l2, l3>;  // one coefficient per (m3, |c|) group
                T g1 = T(0), g2 = T(0);
                static_for<GR::ord.n>([&](auto K) {
                  constexpr cg::Entry en = TI::tab.e[GR::ord.idx[K]];
                  constexpr int pi = en.m1 * n2 + en.m2;
                  if constexpr (kAtUse) {
                    const T xv = x[l1 * l1 + en.m1], av = xa[l1 * l1 + en.m1];
                    const T yv = y[l2 * l2 + en.m2], bv = yb[l2 * l2 + en.m2];
                    if constexpr (GR::ord.open[K]) {
                      g1 = xv * yv;
                      g2 = fmaT(av, yv, xv * bv);
                    } else if constexpr (GR::ord.sub[K]) {
                      g1 = fmaT(-xv, yv, g1);
                      g2 = fmaT(-av, yv, fmaT(-xv, bv, g2));
                    } else {
                      g1 = fmaT(xv, yv, g1);
                      g2 = fmaT(av, yv, fmaT(xv, bv, g2));
                    }
                  } else if constexpr (GR::ord.open[K]) {
                    g1 = p1[pi];
                    g2 = p2[pi];
                  } else if constexpr (GR::ord.sub[K]) {
                    g1 = g1 - p1[pi];
                    g2 = g2 - p2[pi];
                  } else {
                    g1 = g1 + p1[pi];
                    g2 = g2 + p2[pi];
                  }
                  if constexpr (GR::ord.close[K]) {
                    constexpr T c = GR::ord.flip[K] ? T(-en.mag) : T(en.mag);
                    if constexpr (GR::ord.first_m3[K]) {
                      z1[en.m3] = c * g1;
                      z2[en.m3] = c * g2;
                    } else {
                      z1[en.m3] = fmaT(c, g1, z1[en.m3]);
                      z2[en.m3] = fmaT(c, g2, z2[en.m3]);
                    }
                  }
                });
              } else {
                static_for<TI::tab.n>([&](auto K) {
                  constexpr cg::Entry en = TI::tab.e[K];
                  constexpr T c = en.neg ? T(-en.mag) : T(en.mag);
                  constexpr int pi = en.m1 * n2 + en.m2;
                  if constexpr (TI::first_m3(K)) {
                    z1[en.m3] = c * p1[pi];
                    z2[en.m3] = c * p2[pi];
                  } else {
                    z1[en.m3] = fmaT(c, p1[pi], z1[en.m3]);
                    z2[en.m3] = fmaT(c, p2[pi], z2[en.m3]);
                  }
                });
              }
              if (P::template first3<t>(a)) {
                static_for<n3>([&](auto M3) { te[l3 * l3 + M3] = fmaT(w[t], z2[M3], wc[t] * z1[M3]); });
              } else {
                static_for<n3>([&](auto M3) {
                  te[l3 * l3 + M3] = fmaT(w[t], z2[M3], fmaT(wc[t], z1[M3], te[l3 * l3 + M3]));
                });
              }
            }
          }
        });
      });
    });
  }
};

// Rows of a small graph are split over R waves of one block (R = 1: one
// wave per row).  Part p of a row takes a contiguous, slot-aligned range of
// its edges; the parts' fp64 row sums meet in LDS after a block barrier and
// part 0 finishes the row.  Returns this part's [beg, end).
template <int R>
__device__ __forceinline__ void row_part(int beg, int end, int nsl, int part, int& pb, int& pe) {
  if constexpr (R == 1) {
    pb = beg;
    pe = end;
  } else {
    const int steps = (end - beg + nsl - 1) / nsl;
    const int per = (steps + R - 1) / R;
    const int s0 = min(steps, part * per);
    const int s1 = min(steps, s0 + per);
    pb = beg + s0 * nsl;
    pe = min(end, beg + s1 * nsl);
  }
}

// Forward (DD = false): out = the convolution.  Double backward's first pass
// (DD = true): out = grad_G, from the cotangents a (gathered like x), b (like
// Y) and c (like W); a null cotangent reads as zeros.  kYVec: Y of each edge from
// its vector a.vec, evaluated per chunk of kChunk row edges (one lane each)
// into the wave's LDS block s_y.
template <typename T, int L, class P, bool DD, int R, int YS = kYGlobal>
__global__ __launch_bounds__(256) void fwd_kernel(const KernelArgs a) {
  constexpr bool SHV = YS == kYVec;
  constexpr bool kStage = YS != kYGlobal;  // the chunk's Y rows staged in LDS
  static_assert(!(kStage && DD), "staged harmonics: forward only");
  using F = Fwd<T, L, P>;
  using FD = FwdDD<T, L, P>;
  using A = typename RowAcc<T>::type;
  constexpr int NL = F::NL, NT = F::NT;
  static_assert(R == 1 || R == 2 || R == 4, "row split must divide the block's 4 waves");
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int part = wave % R;
  const int wid = blockIdx.x * (4 / R) + wave / R;
  const bool has_row = wid < a.n_rows;
  if constexpr (R == 1) {
    if (!has_row) return;  // wave-uniform
  }
  const int node = has_row ? __builtin_amdgcn_readfirstlane(a.order[wid]) : 0;
  const int lg = P::lps_log2(a);
  const int slot = lane >> lg;
  const int u = lane & ((1 << lg) - 1);
  const bool chan_ok = u < P::mul(a);
  const int uc = chan_ok ? u : 0;  // idle lanes read channel 0 (valid addresses) and never store

  const T* __restrict__ X = static_cast<const T*>(a.x);
  const T* __restrict__ Yp = static_cast<const T*>(a.Y);
  const T* __restrict__ Wp = static_cast<const T*>(a.W);
  const T* __restrict__ XA = static_cast<const T*>(a.xa);
  const T* __restrict__ YB = static_cast<const T*>(a.Yb);
  const T* __restrict__ WC = static_cast<const T*>(a.Wc);
  T* __restrict__ O = static_cast<T*>(a.out);
  const int d_in = P::d_in(a), d_sh = P::d_sh(a);
  const int64_t wstride = P::wstride(a);

  // Row sum.  fp64 data: fp64 registers.  fp32 data: each edge's path sum
  // te is added in fp32 into acc for kFlush edges at a time, and acc is then
  // added into an fp64 row sum kept in LDS (one slab per wave, lane-major),
  // which costs no VGPRs.
  constexpr bool kLdsRow = !std::is_same<T, A>::value || row_sum_in_lds<T, L, DD>();
  constexpr bool kSlab = kLdsRow || R > 1;  // per-wave fp64 row slabs in LDS
  constexpr int kFlush = std::is_same<T, A>::value ? 1 : 4;  // fp64 data: straight into the slab
  __shared__ A s_row[kSlab ? 4 : 1][kSlab ? NL : 1][64];
  A* my_row = &s_row[kSlab ? wave : 0][0][lane];
  T acc[NL];
  static_for<NL>([&](auto I) { acc[I] = T(0); });
  if constexpr (kLdsRow) {
    static_for<NL>([&](auto I) { my_row[I * 64] = A(0); });
  }
  auto flush = [&]() {
    if constexpr (kLdsRow) {
      static_for<L + 1>([&](auto I) {
        constexpr int l = I;
        if (P::out_l(a, l)) {
          static_for<2 * l + 1>([&](auto M) {
            my_row[(l * l + M) * 64] += static_cast<A>(acc[l * l + M]);
            acc[l * l + M] = T(0);
          });
        }
      });
    }
  };

  const int nsl = P::nslots(a);
  int beg, end;
  row_part<R>(has_row ? a.row_ptr[node] : 0, has_row ? a.row_ptr[node + 1] : 0, nsl, part, beg, end);
  // 32 edges per chunk when staging keeps four blocks per CU within the LDS
  constexpr int kChunk = kStage ? 32 : 64;
  __shared__ T s_y[kStage ? 4 : 1][kStage ? kChunk : 1][kStage ? NL : 1];
  const T* __restrict__ VEC = static_cast<const T*>(a.vec);
  // the row's edge ids and neighbours are loaded a chunk at a time, one per
  // lane, and handed to the slots with lane shuffles while the wave is
  // converged
  for (int cb = beg; cb < end; cb += kChunk) {
    const int cn = min(kChunk, end - cb);
    const int my_e = lane < cn ? a.eid[cb + lane] : 0;
    const int my_j = lane < cn ? a.col[cb + lane] : 0;
    if constexpr (kStage) {
      wave_lds_sync();  // the previous chunk's reads of s_y come first
      if (lane < cn) {
        T* yl = &s_y[wave][lane][0];
        if constexpr (SHV) {
          const T* v = VEC + 3 * (int64_t)my_e;
          shx::sh_values<L>(double(v[0]), double(v[1]), double(v[2]),
                            [&](int k, double val) { yl[k] = k < d_sh ? T(val) : T(0); });
        } else {
          const T* yr = Yp + (int64_t)my_e * d_sh;
          static_for<NL>([&](auto I) { yl[I] = I < d_sh ? ldg_stream(yr + I) : T(0); });
        }
      }
      wave_lds_sync();
    }
    const int iters = (cn + nsl - 1) / nsl;
    for (int it = 0; it < iters; ++it) {
    const int q = it * nsl + slot;
    const int e = __shfl(my_e, q & 63, 64);
    const int j = __shfl(my_j, q & 63, 64);
    if (q >= cn) continue;
    T x[NL], y[NL], w[NT];
    auto load_x = [&](const T* __restrict__ base, T (&v)[NL]) {
      const T* xr = base + (int64_t)j * d_in;
      static_for<L + 1>([&](auto I) {
        constexpr int l = I;
        const int off = P::in_off(a, l);
        static_for<2 * l + 1>([&](auto M) {
          if (off >= 0) v[l * l + M] = xr[off + uc * (2 * l + 1) + M];
          else v[l * l + M] = T(0);
        });
      });
    };
    auto load_y = [&](const T* __restrict__ base, T (&v)[NL]) {
      const T* yr = base + (int64_t)e * d_sh;
      static_for<NL>([&](auto I) {
        if (I < d_sh) v[I] = ldg_stream(yr + I);
        else v[I] = T(0);
      });
    };
    load_x(X, x);
    if constexpr (kStage) {
      static_for<NL>([&](auto I) { y[I] = s_y[wave][q][I]; });
    } else {
      load_y(Yp, y);
    }
    load_w<T, L, P>(a, Wp, wstride, uc, e, w);
    T te[NL];
    if constexpr (DD) {
      T xa[NL], yb[NL], wc[NT];
      if (XA != nullptr) load_x(XA, xa);
      else static_for<NL>([&](auto I) { xa[I] = T(0); });
      if (YB != nullptr) load_y(YB, yb);
      else static_for<NL>([&](auto I) { yb[I] = T(0); });
      if (WC != nullptr) load_w<T, L, P>(a, WC, wstride, uc, e, wc);
      else static_for<NT>([&](auto I) { wc[I] = T(0); });
      FD::edge(a, __builtin_amdgcn_readfirstlane(e), x, xa, y, yb, w, wc, te);
    } else {
      F::edge(a, __builtin_amdgcn_readfirstlane(e), x, y, w, te);
    }
    static_for<L + 1>([&](auto I) {
      constexpr int l = I;
      if (P::out_l(a, l)) {
        static_for<2 * l + 1>([&](auto M) { acc[l * l + M] += te[l * l + M]; });
      }
    });
    if (it % kFlush == kFlush - 1) flush();
    }
  }
  flush();

  A tot[NL];
  static_for<NL>([&](auto I) {
    if constexpr (kLdsRow) tot[I] = my_row[I * 64];
    else tot[I] = acc[I];
  });
  if constexpr (R > 1) {
    // the row's parts meet in LDS; part 0 finishes the row
    if constexpr (!kLdsRow) {
      static_for<NL>([&](auto I) { my_row[I * 64] = tot[I]; });
    }
    __syncthreads();
    if (part != 0 || !has_row) return;
    static_for<R - 1>([&](auto Q) {
      static_for<NL>([&](auto I) { tot[I] += my_row[(int(Q) + 1) * NL * 64 + I * 64]; });
    });
  }

  // sum the slots' partial rows: slots sit at lane offsets 2^lg .. 32
  for (int off = 1 << lg; off < 64; off <<= 1) {
    static_for<NL>([&](auto I) { tot[I] += __shfl_xor(tot[I], off, 64); });
  }
  if (slot == 0 && chan_ok) {
    T* orow = O + (int64_t)node * P::d_out(a);
    static_for<L + 1>([&](auto I) {
      constexpr int l = I;
      const int off = P::out_off(a, l);
      if (off >= 0) {
        static_for<2 * l + 1>([&](auto M) {
          T* o = &orow[off + u * (2 * l + 1) + M];
          if constexpr (P::kFull) {
            *o = static_cast<T>(tot[l * l + M]);
          } else {  // a plan's later pass adds into what an earlier one wrote
            *o = (a.acc & 1) ? static_cast<T>(static_cast<A>(*o) + tot[l * l + M]) : static_cast<T>(tot[l * l + M]);
          }
        });
      }
    });
  }
}

// ----------------------------------------------------------------- backward
template <typename T, int L, class P>
struct Bwd {
  static constexpr int NL = (L + 1) * (L + 1);
  static constexpr int NT = triple_count(L);

  // A path with an l = 0 leg (one coefficient c for every m, TabInfo::kDiag):
  //   (l, 0, l): d = x . G[l3];  dW = c Y0 d;  dx += (W c Y0) G;  dY0 += W c d
  //   (0, l, l): d = G . Y[l2];  dW = c x0 d;  dx0 += W c d;     dY += (W c x0) G
  //   (l, l, 0): s = c G0;       dW = s x.Y;   dx += (W s) Y;    dY += (W s) x
  // The per-entry products of the general case are not formed.
  template <int l1, int l2, int l3, int NV>
  static __device__ __forceinline__ void diag_path(T w, const T (&x)[NL], const T (&y)[NL], const T (&g)[NL],
                                                   T (&dxe)[NL], T (&dya)[NV], bool first1, bool store_dw,
                                                   T* dw_at) {
    using TI = TabInfo<l1, l2, l3>;
    constexpr T c = T(TI::kDiagCoef);
    constexpr int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1;
    auto add_dx = [&](T f, auto src_at) {
      static_for<n1>([&](auto M) {
        if (first1) dxe[l1 * l1 + M] = f * src_at(M);
        else dxe[l1 * l1 + M] = fmaT(f, src_at(M), dxe[l1 * l1 + M]);
      });
    };
    if constexpr (TI::kDiag == 1) {
      T d = x[l1 * l1] * g[l3 * l3];
      static_for<n1 - 1>([&](auto M) { d = fmaT(x[l1 * l1 + M + 1], g[l3 * l3 + M + 1], d); });
      const T cy = c * y[0];
      if (store_dw) __builtin_nontemporal_store(cy * d, dw_at);
      add_dx(w * cy, [&](int m) { return g[l3 * l3 + m]; });
      dya[0] = fmaT(w, c * d, dya[0]);
    } else if constexpr (TI::kDiag == 2) {
      T d = g[l3 * l3] * y[l2 * l2];
      static_for<n2 - 1>([&](auto M) { d = fmaT(g[l3 * l3 + M + 1], y[l2 * l2 + M + 1], d); });
      const T cd = c * d;
      if (store_dw) __builtin_nontemporal_store(x[0] * cd, dw_at);
      add_dx(w * cd, [&](int) { return T(1); });
      const T f = w * (c * x[0]);
      static_for<n2>([&](auto M) { dya[l2 * l2 + M] = fmaT(f, g[l3 * l3 + M], dya[l2 * l2 + M]); });
    } else {
      const T s = c * g[l3 * l3];
      T d = x[l1 * l1] * y[l2 * l2];
      static_for<n1 - 1>([&](auto M) { d = fmaT(x[l1 * l1 + M + 1], y[l2 * l2 + M + 1], d); });
      if (store_dw) __builtin_nontemporal_store(s * d, dw_at);
      const T f = w * s;
      add_dx(f, [&](int m) { return y[l2 * l2 + m]; });
      static_for<n2>([&](auto M) { dya[l2 * l2 + M] = fmaT(f, x[l1 * l1 + M], dya[l2 * l2 + M]); });
    }
  }

  // One edge: dW for every path, the edge's contribution dxe to dx (summed
  // over its paths), and per-lane contributions to dY (summed over channels
  // afterwards).
  template <int NV>
  static __device__ __forceinline__ void edge(const KernelArgs& a, int tok, const T (&x)[NL], const T (&y)[NL],
                                              const T (&g)[NL], const T (&w)[NT], T (&dxe)[NL],
                                              T (&dya)[NV], bool store_dw, T* dwr) {
    static_assert(NV >= NL, "dY accumulator too short");
    static_for<L + 1>([&](auto I3) {
      constexpr int l3 = I3;
      static_for<L + 1>([&](auto I1) {
        constexpr int l1 = I1;
        static_for<L + 1>([&](auto I2) {
          constexpr int l2 = I2;
          if constexpr (cg::triangle(l1, l2, l3) && triple_in_class(l1, l2, l3, P::kPar)) {
            constexpr int t = triple_id(L, l1, l2, l3);
            if (P::template on<t>(a) && P::template run<t>(a, tok)) {
              using TI = TabInfo<l1, l2, l3>;
              constexpr int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1;
              if constexpr (TI::kDiag != 0) {
                diag_path<l1, l2, l3>(w[t], x, y, g, dxe, dya, P::template first1<t>(a), store_dw,
                                      dwr + P::template woff<t>(a));
                return;
              }
              T dxp[n1], dyp[n2];
              static_for<TI::tab.n>([&](auto K) {
                constexpr cg::Entry en = TI::tab.e[K];
                constexpr T mag = T(en.mag);
                const T cgm = mag * g[l3 * l3 + en.m3];  // shared by entries with equal |c| and m3
                const T cgs = en.neg ? -cgm : cgm;
                if constexpr (TI::first_m1(K))
                  dxp[en.m1] = cgs * y[l2 * l2 + en.m2];
                else
                  dxp[en.m1] = fmaT(cgs, y[l2 * l2 + en.m2], dxp[en.m1]);
                if constexpr (TI::first_m2(K))
                  dyp[en.m2] = cgs * x[l1 * l1 + en.m1];
                else
                  dyp[en.m2] = fmaT(cgs, x[l1 * l1 + en.m1], dyp[en.m2]);
              });
              T s = T(0);
              static_for<n1>([&](auto M1) {
                if constexpr (TI::has_m1(M1)) s = fmaT(x[l1 * l1 + M1], dxp[M1], s);
              });
              if (store_dw) __builtin_nontemporal_store(s, dwr + P::template woff<t>(a));
              if (P::template first1<t>(a)) {
                static_for<n1>([&](auto M1) {
                  if constexpr (TI::has_m1(M1))
                    dxe[l1 * l1 + M1] = w[t] * dxp[M1];
                  else
                    dxe[l1 * l1 + M1] = T(0);
                });
              } else {
                static_for<n1>([&](auto M1) {
                  if constexpr (TI::has_m1(M1)) dxe[l1 * l1 + M1] = fmaT(w[t], dxp[M1], dxe[l1 * l1 + M1]);
                });
              }
              static_for<n2>([&](auto M2) {
                if constexpr (TI::has_m2(M2)) dya[l2 * l2 + M2] = fmaT(w[t], dyp[M2], dya[l2 * l2 + M2]);
              });
            }
          }
        });
      });
    });
  }
};

// Double backward, second pass (source-sorted rows).  With a, b, c the
// cotangents of grad_x, grad_Y, grad_W, per path:
//   dxp = CG(., Y, G), dxq = CG(., b, G), xt = W a + c x, dyt = CG(xt, ., G)
//   grad_W[p,u]   = a . dxp + x . dxq            (stored at once, or with kLate
//                                                 returned and stored by the caller)
//   grad_x (row) += W dxq + c dxp
//   grad_Y (lane)+= dyt                          (summed over channels later)
// Each nonzero costs three FMAs sharing one product |c| * G[m3]; folding the
// weights into xt first saves the fourth (grad_Y = CG(W a + c x, ., G)).
template <typename T, int L, class P>
struct BwdDD {
  static constexpr int NL = (L + 1) * (L + 1);
  static constexpr int NT = triple_count(L);

  // A path with an l = 0 leg (one coefficient k for every m, TabInfo::kDiag;
  // C the weight cotangent); S is the grad_W value, returned:
  //   (l, 0, l): dA = a . G, dX = x . G;  S = k (Y0 dA + b0 dX)
  //              grad_x += k (W b0 + C Y0) G;           grad_Y0 += k (W dA + C dX)
  //   (0, l, l): dY = G . Y, dB = G . b;  S = k (a0 dY + x0 dB)
  //              grad_x0 += k (W dB + C dY);            grad_Y += k (W a0 + C x0) G
  //   (l, l, 0): s = k G0, d = a . Y + x . b;  S = s d
  //              grad_x += (W s) b + (C s) Y;           grad_Y += (W s) a + (C s) x
  template <int l1, int l2, int l3, int NV, class XR>
  static __device__ __forceinline__ T diag_path(T w, T wc, const XR& x, const XR& xa, const T (&y)[NL],
                                                const T (&yb)[NL], const T (&g)[NL], T (&dxe)[NL], T (&dya)[NV],
                                                bool first1) {
    using TI = TabInfo<l1, l2, l3>;
    constexpr T c = T(TI::kDiagCoef);
    constexpr int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1;
    if constexpr (TI::kDiag == 1) {
      T dA = xa[l1 * l1] * g[l3 * l3], dX = x[l1 * l1] * g[l3 * l3];
      static_for<n1 - 1>([&](auto M) {
        dA = fmaT(xa[l1 * l1 + M + 1], g[l3 * l3 + M + 1], dA);
        dX = fmaT(x[l1 * l1 + M + 1], g[l3 * l3 + M + 1], dX);
      });
      const T f = c * fmaT(w, yb[0], wc * y[0]);
      static_for<n1>([&](auto M) {
        if (first1) dxe[l1 * l1 + M] = f * g[l3 * l3 + M];
        else dxe[l1 * l1 + M] = fmaT(f, g[l3 * l3 + M], dxe[l1 * l1 + M]);
      });
      dya[0] = fmaT(c, fmaT(w, dA, wc * dX), dya[0]);
      return c * fmaT(y[0], dA, yb[0] * dX);
    } else if constexpr (TI::kDiag == 2) {
      T dY = g[l3 * l3] * y[l2 * l2], dB = g[l3 * l3] * yb[l2 * l2];
      static_for<n2 - 1>([&](auto M) {
        dY = fmaT(g[l3 * l3 + M + 1], y[l2 * l2 + M + 1], dY);
        dB = fmaT(g[l3 * l3 + M + 1], yb[l2 * l2 + M + 1], dB);
      });
      const T f0 = c * fmaT(w, dB, wc * dY);
      if (first1) dxe[0] = f0;
      else dxe[0] = dxe[0] + f0;
      const T f = c * fmaT(w, xa[0], wc * x[0]);
      static_for<n2>([&](auto M) { dya[l2 * l2 + M] = fmaT(f, g[l3 * l3 + M], dya[l2 * l2 + M]); });
      return c * fmaT(xa[0], dY, x[0] * dB);
    } else {
      const T sg = c * g[l3 * l3];
      T d = x[l1 * l1] * yb[l2 * l2];
      d = fmaT(xa[l1 * l1], y[l2 * l2], d);
      static_for<n1 - 1>([&](auto M) {
        d = fmaT(xa[l1 * l1 + M + 1], y[l2 * l2 + M + 1], d);
        d = fmaT(x[l1 * l1 + M + 1], yb[l2 * l2 + M + 1], d);
      });
      const T f1 = w * sg, f2 = wc * sg;
      static_for<n1>([&](auto M) {
        if (first1) dxe[l1 * l1 + M] = fmaT(f1, yb[l2 * l2 + M], f2 * y[l2 * l2 + M]);
        else dxe[l1 * l1 + M] = fmaT(f1, yb[l2 * l2 + M], fmaT(f2, y[l2 * l2 + M], dxe[l1 * l1 + M]));
      });
      static_for<n2>([&](auto M) {
        dya[l2 * l2 + M] = fmaT(f1, xa[l1 * l1 + M], fmaT(f2, x[l1 * l1 + M], dya[l2 * l2 + M]));
      });
      return sg * d;
    }
  }

  template <bool kLate, int NV, class XR>
  static __device__ __forceinline__ void edge(const KernelArgs& a, int tok, const XR& x, const XR& xa,
                                              const T (&y)[NL], const T (&yb)[NL], const T (&g)[NL],
                                              const T (&w)[NT], const T (&wc)[NT], T (&dxe)[NL], T (&dya)[NV],
                                              bool store_dw, T* dwr, T (&dwv)[NT]) {
    static_assert(NV >= NL, "dY accumulator too short");
    static_for<L + 1>([&](auto I3) {
      constexpr int l3 = I3;
      static_for<L + 1>([&](auto I1) {
        constexpr int l1 = I1;
        static_for<L + 1>([&](auto I2) {
          constexpr int l2 = I2;
          if constexpr (cg::triangle(l1, l2, l3) && triple_in_class(l1, l2, l3, P::kPar)) {
            constexpr int t = triple_id(L, l1, l2, l3);
            if (P::template on<t>(a) && P::template run<t>(a, tok)) {
              using TI = TabInfo<l1, l2, l3>;
              constexpr int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1;
              if constexpr (TI::kDiag != 0) {
                const T sd = diag_path<l1, l2, l3>(w[t], wc[t], x, xa, y, yb, g, dxe, dya, P::template first1<t>(a));
                if constexpr (kLate)
                  dwv[t] = sd;
                else if (store_dw)
                  __builtin_nontemporal_store(sd, dwr + P::template woff<t>(a));
                return;
              }
              T dxp[n1], dxq[n1], xt[n1], dyt[n2];
              static_for<n1>([&](auto M1) {
                if constexpr (TI::has_m1(M1)) xt[M1] = fmaT(w[t], xa[l1 * l1 + M1], wc[t] * x[l1 * l1 + M1]);
              });
              static_for<TI::tab.n>([&](auto K) {
                constexpr cg::Entry en = TI::tab.e[K];
                constexpr T mag = T(en.mag);
                const T cgm = mag * g[l3 * l3 + en.m3];
                const T cgs = en.neg ? -cgm : cgm;
                const T yv = y[l2 * l2 + en.m2], bv = yb[l2 * l2 + en.m2];
                if constexpr (TI::first_m1(K)) {
                  dxp[en.m1] = cgs * yv;
                  dxq[en.m1] = cgs * bv;
                } else {
                  dxp[en.m1] = fmaT(cgs, yv, dxp[en.m1]);
                  dxq[en.m1] = fmaT(cgs, bv, dxq[en.m1]);
                }
                if constexpr (TI::first_m2(K))
                  dyt[en.m2] = cgs * xt[en.m1];
                else
                  dyt[en.m2] = fmaT(cgs, xt[en.m1], dyt[en.m2]);
              });
              T s = T(0);
              static_for<n1>([&](auto M1) {
                if constexpr (TI::has_m1(M1)) {
                  s = fmaT(xa[l1 * l1 + M1], dxp[M1], s);
                  s = fmaT(x[l1 * l1 + M1], dxq[M1], s);
                }
              });
              if constexpr (kLate)
                dwv[t] = s;
              else if (store_dw)
                __builtin_nontemporal_store(s, dwr + P::template woff<t>(a));
              if (P::template first1<t>(a)) {
                static_for<n1>([&](auto M1) {
                  if constexpr (TI::has_m1(M1))
                    dxe[l1 * l1 + M1] = fmaT(w[t], dxq[M1], wc[t] * dxp[M1]);
                  else
                    dxe[l1 * l1 + M1] = T(0);
                });
              } else {
                static_for<n1>([&](auto M1) {
                  if constexpr (TI::has_m1(M1))
                    dxe[l1 * l1 + M1] = fmaT(w[t], dxq[M1], fmaT(wc[t], dxp[M1], dxe[l1 * l1 + M1]));
                });
              }
              static_for<n2>([&](auto M2) {
                if constexpr (TI::has_m2(M2)) dya[l2 * l2 + M2] += dyt[M2];
              });
            }
          }
        });
      });
    });
  }
};

// Per-edge inputs of the backward kernels: G row of the destination, the
// edge's Y row and weights, and for the double backward the cotangents b
// (like Y) and c (like W).
template <typename T, int L, bool DD>
struct EdgeIn {
  static constexpr int NL = (L + 1) * (L + 1);
  static constexpr int NT = triple_count(L);
  T g[NL], y[NL], w[NT];
  T yb[DD ? NL : 1], wc[DD ? NT : 1];
};

constexpr int pow2_ceil(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

// The backward keeps a second set of edge-input registers (one edge ahead)
// where that still fits in 256 VGPRs: fp32 up to l = 2, and l = 3 with the
// even-parity path set.  Wider kernels already spill to AGPRs with one set,
// and a second would double that.
template <typename T, int L, class P, bool DD>
constexpr bool bwd_pipelined() {
  return !DD && sizeof(T) == 4 && (L <= 2 || (L == 3 && P::kPar == kEvenOnly));
}

// Backward (DD = false): grad_x (out), grad_Y (dY), grad_W (dW) of <G, out>.
// Double backward's second pass (DD = true): the same three outputs of
// <a, dx> + <b, dY> + <c, dW>, with the cotangents a (row-resident like x),
// b and c; a null cotangent reads as zeros.  kYVec: Y from the edge vectors
// a.vec per chunk of 64 row edges (as in the forward), each edge's
// channel-summed dY into the wave's LDS block, and at the chunk's end
// grad_vec (a.gvec) of its edges, one lane each.
template <typename T, int L, class P, bool DD, int R, int YS = kYGlobal>
__global__ __launch_bounds__(256) void bwd_kernel(const KernelArgs a) {
  constexpr bool SHV = YS == kYVec;
  static_assert(YS != kYRows, "the backward loads Y per slot or evaluates it from vectors");
  static_assert(!(SHV && DD), "harmonics from edge vectors: backward only");
  using B = Bwd<T, L, P>;
  using BD = BwdDD<T, L, P>;
  using In = EdgeIn<T, L, DD>;
  using A = typename RowAcc<T>::type;
  constexpr int NL = B::NL, NT = B::NT;
  constexpr int NV = pow2_ceil(NL);  // dY values, padded to a power of two for the reduce-scatter
  static_assert(R == 1 || R == 2 || R == 4, "row split must divide the block's 4 waves");
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int part = wave % R;
  const int wid = blockIdx.x * (4 / R) + wave / R;
  const bool has_row = wid < a.n_rows;
  if constexpr (R == 1) {
    if (!has_row) return;  // wave-uniform
  }
  const int node = has_row ? __builtin_amdgcn_readfirstlane(a.order[wid]) : 0;
  const int lg = P::lps_log2(a);
  const int lps = 1 << lg;
  const int slot = lane >> lg;
  const int u = lane & (lps - 1);
  const bool chan_ok = u < P::mul(a);
  const int uc = chan_ok ? u : 0;

  const T* __restrict__ X = static_cast<const T*>(a.x);
  const T* __restrict__ Yp = static_cast<const T*>(a.Y);
  const T* __restrict__ Wp = static_cast<const T*>(a.W);
  const T* __restrict__ Gp = static_cast<const T*>(a.G);
  T* __restrict__ DX = static_cast<T*>(a.out);
  T* __restrict__ DY = static_cast<T*>(a.dY);
  T* __restrict__ DW = static_cast<T*>(a.dW);
  const T* __restrict__ XA = static_cast<const T*>(a.xa);
  const T* __restrict__ YB = static_cast<const T*>(a.Yb);
  const T* __restrict__ WC = static_cast<const T*>(a.Wc);
  const int d_out = P::d_out(a), d_sh = P::d_sh(a);
  const int64_t wstride = P::wstride(a);
  const T* __restrict__ VEC = static_cast<const T*>(a.vec);
  T* __restrict__ GV = static_cast<T*>(a.gvec);
  // kYVec: per wave, the current chunk's harmonics and channel-summed dY (row
  // position within the chunk major), and the vectors and edge ids of the
  // chunk by its parity (a chunk's ids are fetched one step before the
  // previous chunk's last step has run)
  __shared__ T s_vy[SHV ? 4 : 1][SHV ? 64 : 1][SHV ? NL : 1];
  __shared__ T s_vdy[SHV ? 4 : 1][SHV ? 64 : 1][SHV ? NL : 1];
  __shared__ T s_vv[SHV ? 4 : 1][SHV ? 2 : 1][SHV ? 64 : 1][SHV ? 3 : 1];
  __shared__ int s_ve[SHV ? 4 : 1][SHV ? 2 : 1][SHV ? 64 : 1];

  // this source node's features (and for the double backward its cotangent
  // a) stay in registers for the whole row; idle lanes hold zeros so they
  // add nothing to the channel sums of dY
  auto load_row = [&](const T* __restrict__ base, bool present, T (&v)[NL]) {
    const T* xr = base + (int64_t)node * P::d_in(a);
    static_for<L + 1>([&](auto I) {
      constexpr int l = I;
      const int off = P::in_off(a, l);
      static_for<2 * l + 1>([&](auto M) {
        if (off >= 0 && chan_ok && present) v[l * l + M] = xr[off + u * (2 * l + 1) + M];
        else v[l * l + M] = T(0);
      });
    });
    // wait for the row here, before any dW / dY store is in flight
    static_for<NL>([&](auto I) { pin_vgpr(v[I]); });
  };
  // For the fp64 l >= 4 double backward the row's x and a live in a per-wave
  // LDS slab (lane-major) instead of registers: its per-edge state otherwise
  // spills to scratch, and the spills reached HBM.  (Whole rows only: the
  // split-row kernels need their LDS to combine the row.)
  constexpr bool kXLds = DD && sizeof(T) == 8 && L >= 4 && R == 1;
  __shared__ T s_xrow[kXLds ? 4 : 1][2][kXLds ? NL : 1][64];
  T x[kXLds ? 1 : NL];
  T xa[(DD && !kXLds) ? NL : 1];
  if constexpr (kXLds) {
    T t[NL];
    load_row(X, true, t);
    static_for<NL>([&](auto I) { s_xrow[wave][0][I][lane] = t[I]; });
    load_row(XA, XA != nullptr, t);
    static_for<NL>([&](auto I) { s_xrow[wave][1][I][lane] = t[I]; });
  } else {
    load_row(X, true, x);
    if constexpr (DD) load_row(XA, XA != nullptr, xa);
  }
  struct LdsRow {
    const T* p;
    __device__ __forceinline__ T operator[](int i) const { return p[i * 64]; }
  };
  // The fp32 l = 3 double backward over whole rows with a compile-time
  // table (kLate) keeps an edge's grad_W and grad_Y values until the next
  // edge's loads are issued (store_pending below): those loads then sit
  // ahead of the stores in the in-order memory counter, and waiting for them
  // does not wait for this edge's stores.  Everything else stores at once:
  // fp64 l = 4 measured slower (twice the registers held), the split-row
  // and run-time-table kernels drop to one wave per SIMD, and at other l the
  // compiler waits for all stores more often, not less.
  constexpr bool kLate = DD && sizeof(T) == 4 && L == 3 && P::kFull && R == 1;
  // dx row sum: registers, or a per-wave LDS slab, lane-major, for kLate
  // (room for the held values) and for the fp64 l = 4 double backward (whose
  // per-edge state spills to scratch otherwise).  The plain backward,
  // fp64 l = 4 included, measured slower with the slab.
  constexpr bool kDxLds = kLate || (DD && sizeof(T) == 8 && L >= 4);
  __shared__ A s_dxrow[kDxLds ? 4 : 1][kDxLds ? NL : 1][64];
  A* const my_dx = &s_dxrow[kDxLds ? wave : 0][0][lane];
  A dxa[NL];
  static_for<NL>([&](auto I) {
    if constexpr (kDxLds) my_dx[I * 64] = A(0);
    else dxa[I] = A(0);
  });

  // The wave walks the row in steps of nslots edges: step k gives slot s the
  // edge at row position k * nslots + s.  Edge ids arrive 64 at a time (one
  // per lane) and are handed to the slots with lane shuffles.  The inputs of
  // step k + 1 are requested before step k computes and stores, so their
  // latency hides behind step k and the in-order memory counter never has to
  // wait for this step's dW / dY stores before the next step can start.
  int beg, pend;
  row_part<R>(has_row ? a.row_ptr[node] : 0, has_row ? a.row_ptr[node + 1] : 0, 64 >> lg, part, beg, pend);
  const int deg = pend - beg;                   // this part's edges of the row
  const int lgs = 6 - lg;                       // log2(slots per wave)
  const int n_steps = (deg + (1 << lgs) - 1) >> lgs;
  const int chunk_mask = (64 >> lgs) - 1;       // steps per chunk of 64 ids, minus one
  int my_e = 0, my_i = 0;
  auto fetch_ids = [&](int k) {
    const int p = (k << lgs) + lane;
    my_e = p < deg ? a.eid[beg + p] : 0;
    my_i = p < deg ? a.col[beg + p] : 0;
    // wait for the ids here: a wait at their first use inside the loop
    // would also wait for every store still in flight
    pin_vgpr(my_e);
    pin_vgpr(my_i);
    if constexpr (SHV) {
      // this chunk's harmonics, one lane per edge; lanes past the row's end
      // take a zero vector (Y = (1, 0, ...)), so every entry is defined
      const int par = (k >> lg) & 1;
      double vx = 0.0, vy = 0.0, vz = 0.0;
      if (p < deg) {
        const T* v = VEC + 3 * (int64_t)my_e;
        vx = double(v[0]);
        vy = double(v[1]);
        vz = double(v[2]);
      }
      wave_lds_sync();  // the previous chunk's reads of s_vy come first
      T* yl = &s_vy[wave][lane][0];
      shx::sh_values<L>(vx, vy, vz, [&](int kk, double val) { yl[kk] = kk < d_sh ? T(val) : T(0); });
      s_vv[wave][par][lane][0] = T(vx);
      s_vv[wave][par][lane][1] = T(vy);
      s_vv[wave][par][lane][2] = T(vz);
      s_ve[wave][par][lane] = my_e;
      wave_lds_sync();
    }
  };
  auto load_y = [&](const T* __restrict__ base, bool present, int e, T (&y)[NL]) {
    const T* yr = base + (int64_t)e * d_sh;
    static_for<NL>([&](auto I) {
      if (I < d_sh && present) y[I] = ldg_stream(yr + I);
      else y[I] = T(0);
    });
  };
  auto load_wrow = [&](const T* __restrict__ base, bool present, int e, T (&w)[NT]) {
    const T* wr = base + (int64_t)e * wstride + uc;
    static_for<NT>([&](auto I) {
      constexpr TripleInfo ti = triple_at(L, I);
      if constexpr (triple_in_class(ti.l1, ti.l2, ti.l3, P::kPar)) {
        if (P::template on<I>(a) && present) w[I] = ldg_stream(wr + P::template woff<I>(a));
        else w[I] = T(0);
      } else {
        w[I] = T(0);
      }
    });
  };
  auto load_edge = [&](int e, int i, int q, In& in) {
    const T* gr = Gp + (int64_t)i * d_out;
    static_for<L + 1>([&](auto I) {
      constexpr int l = I;
      const int off = P::out_off(a, l);
      static_for<2 * l + 1>([&](auto M) {
        if (off >= 0) in.g[l * l + M] = gr[off + uc * (2 * l + 1) + M];
        else in.g[l * l + M] = T(0);
      });
    });
    if constexpr (SHV) {
      static_for<NL>([&](auto I) { in.y[I] = s_vy[wave][q][I]; });
    } else {
      load_y(Yp, true, e, in.y);
    }
    load_wrow(Wp, true, e, in.w);
    if constexpr (DD) {
      load_y(YB, YB != nullptr, e, in.yb);
      load_wrow(WC, WC != nullptr, e, in.wc);
    }
  };

  // Two register sets for the edge inputs, used alternately, so the step
  // that prefetches into one set never copies registers still being loaded.
  // Loads and arithmetic run unconditionally: a slot past the end of the row
  // reads edge 0 / node 0 (its ids are 0) and only its stores and its share
  // of dx are masked, which keeps every load out of divergent control flow.
  auto prefetch = [&](int k, int& e, bool& valid, int& q, In& in) {
    const int r = k & chunk_mask;
    if (r == 0) fetch_ids(k);
    q = (r << lgs) + slot;  // position within the chunk
    e = __shfl(my_e, q, 64);
    const int i = __shfl(my_i, q, 64);
    valid = (k << lgs) + slot < deg;
    load_edge(e, i, q, in);
  };
  struct Pending {
    T dw[NT];  // unused, and removed, unless kLate
    T dy[kLate ? NV : 1];
    int base, nv;
  };
  auto compute = [&](const int e, const bool valid, const int q, const In& in, Pending& pd) {
    T dya[NV], dxe[NL];
    static_for<NV>([&](auto I) { dya[I] = T(0); });
    // idle lanes (u >= U) aim their dW stores at channel 0 of the same row
    // and store only when chan_ok; for a power-of-two U every lane is active
    const bool store_dw = DW != nullptr;
    T* dwr = store_dw ? DW + (int64_t)e * wstride + uc : nullptr;
    const bool st = store_dw && chan_ok && valid;
    if constexpr (DD && kXLds)
      BD::template edge<kLate>(a, __builtin_amdgcn_readfirstlane(e), LdsRow{&s_xrow[wave][0][0][lane]},
                               LdsRow{&s_xrow[wave][1][0][lane]}, in.y, in.yb, in.g, in.w, in.wc, dxe, dya, st, dwr,
                               pd.dw);
    else if constexpr (DD)
      BD::template edge<kLate>(a, __builtin_amdgcn_readfirstlane(e), x, xa, in.y, in.yb, in.g, in.w, in.wc, dxe,
                               dya, st, dwr, pd.dw);
    else
      B::edge(a, __builtin_amdgcn_readfirstlane(e), x, in.y, in.g, in.w, dxe, dya, st, dwr);
    static_for<L + 1>([&](auto I) {
      constexpr int l = I;
      if (P::in_l(a, l)) {
        static_for<2 * l + 1>([&](auto M) {
          const A v = valid ? static_cast<A>(dxe[l * l + M]) : A(0);
          if constexpr (kDxLds) my_dx[(l * l + M) * 64] += v;
          else dxa[l * l + M] += v;
        });
      }
    });

    if (SHV ? GV != nullptr : DY != nullptr) {
      // reduce-scatter of the NV dY values over the slot's lanes.  Step s
      // pairs lanes across bit b = lps >> (s+1); while more than one value is
      // left, lanes with bit b set keep the upper half, the others the lower.
      int base = 0;
      int nv = NV;
      static_for<6>([&](auto S) {
        constexpr int s = S;
        const int b = lps >> (s + 1);
        if (b >= 1) {
          if constexpr ((NV >> s) > 1) {
            constexpr int h = NV >> (s + 1);
            const bool upper = (u & b) != 0;
            static_for<h>([&](auto V) {
              // opaque copies: a select between two array elements could be
              // folded into one load with a run-time index, which would move
              // the whole array to LDS
              T lo = dya[V], hi = dya[V + h];
              pin_vgpr(lo);
              pin_vgpr(hi);
              const T keep = upper ? hi : lo;
              const T send = upper ? lo : hi;
              dya[V] = keep + __shfl_xor(send, b, 64);
            });
            if (upper) base += h;
            nv = h;
          } else {
            dya[0] += __shfl_xor(dya[0], b, 64);
          }
        }
      });
      if constexpr (kLate) {
        static_for<NV>([&](auto V) { pd.dy[V] = dya[V]; });
        pd.base = base;
        pd.nv = nv;
      } else if constexpr (SHV) {
        const int plain_mask = lps > NV ? lps / NV - 1 : 0;
        if ((u & plain_mask) == 0 && valid) {
          static_for<NV>([&](auto J) {
            if (J < nv && base + J < d_sh) s_vdy[wave][q][base + J] = dya[J];
          });
        }
      } else {
        // bits below lps/NV were plain sums: one lane of each such group stores
        const int plain_mask = lps > NV ? lps / NV - 1 : 0;
        if ((u & plain_mask) == 0 && valid) {
          T* dyr = DY + (int64_t)e * d_sh;
          static_for<NV>([&](auto V) {
            if (V < nv && base + V < d_sh) {
              if constexpr (P::kFull) dyr[base + V] = dya[V];
              else dyr[base + V] = (a.acc & 2) ? dyr[base + V] + dya[V] : dya[V];
            }
          });
        }
      }
    }
  };
  auto store_pending = [&](const int e, const bool valid, const Pending& pd) {
    if constexpr (kLate) {
      if (DW != nullptr && chan_ok && valid) {
        T* dwr = DW + (int64_t)e * wstride + uc;
        static_for<NT>([&](auto I) {
          constexpr TripleInfo ti = triple_at(L, I);
          if constexpr (triple_in_class(ti.l1, ti.l2, ti.l3, P::kPar)) {
            if (P::template on<I>(a)) __builtin_nontemporal_store(pd.dw[I], dwr + P::template woff<I>(a));
          }
        });
      }
      if (DY != nullptr) {
        const int plain_mask = lps > NV ? lps / NV - 1 : 0;
        if ((u & plain_mask) == 0 && valid) {
          T* dyr = DY + (int64_t)e * d_sh;
          static_for<NV>([&](auto V) {
            if (V < pd.nv && pd.base + V < d_sh) dyr[pd.base + V] = pd.dy[V];
          });
        }
      }
    }
  };

  // kYVec: after a chunk's last step, grad_vec of the chunk's edges (one lane
  // each) from their vectors and channel-summed dY in LDS
  auto chunk_pass = [&](int k) {
    if constexpr (SHV) {
      if (GV == nullptr) return;
      if (((k + 1) & chunk_mask) != 0 && k + 1 < n_steps) return;  // wave-uniform
      wave_lds_sync();  // the chunk's dY writes come first
      const int par = (k >> lg) & 1;
      const int pos = ((k >> lg) << 6) + lane;  // this lane's row position in the chunk
      if (pos < deg) {
        const int e = s_ve[wave][par][lane];
        const T* gy = &s_vdy[wave][lane][0];
        const T* vv = &s_vv[wave][par][lane][0];
        double gx, gyv, gz;
        shx::sh_vec_grad<L>(double(vv[0]), double(vv[1]), double(vv[2]),
                            [&](int kk) { return kk < d_sh ? double(gy[kk]) : 0.0; }, gx, gyv, gz);
        T* o = GV + 3 * (int64_t)e;
        o[0] = T(gx);
        o[1] = T(gyv);
        o[2] = T(gz);
      }
      wave_lds_sync();  // and the next chunk's dY writes after these reads
    }
  };

  In ia;
  int ea = 0, qa = 0;
  bool va = false;
  Pending pd;
  if constexpr (bwd_pipelined<T, L, P, DD>()) {
    In ib;
    int eb = 0, qb = 0;
    bool vb = false;
    if (n_steps > 0) prefetch(0, ea, va, qa, ia);
    for (int k = 0; k < n_steps; k += 2) {  // wave-uniform trip count
      prefetch(k + 1, eb, vb, qb, ib);
      compute(ea, va, qa, ia, pd);
      chunk_pass(k);
      if (k + 1 >= n_steps) break;
      prefetch(k + 2, ea, va, qa, ia);
      compute(eb, vb, qb, ib, pd);
      chunk_pass(k + 1);
    }
  } else if constexpr (kLate) {
    if (n_steps > 0) prefetch(0, ea, va, qa, ia);
    for (int k = 0; k < n_steps; ++k) {  // wave-uniform trip count
      compute(ea, va, qa, ia, pd);
      const int e_done = ea;
      const bool v_done = va;
      if (k + 1 < n_steps) prefetch(k + 1, ea, va, qa, ia);
      store_pending(e_done, v_done, pd);
    }
  } else {
    for (int k = 0; k < n_steps; ++k) {
      prefetch(k, ea, va, qa, ia);
      compute(ea, va, qa, ia, pd);
      chunk_pass(k);
    }
  }

  if constexpr (kDxLds) {
    static_for<NL>([&](auto I) { dxa[I] = my_dx[I * 64]; });
  }
  if constexpr (R > 1) {
    // the row's parts meet in LDS; part 0 finishes dx
    __shared__ A s_dx[4][NL][64];
    if (DX != nullptr) {
      static_for<NL>([&](auto I) { s_dx[wave][I][lane] = dxa[I]; });
    }
    __syncthreads();
    if (part != 0 || !has_row) return;
    if (DX != nullptr) {
      static_for<R - 1>([&](auto Q) {
        static_for<NL>([&](auto I) { dxa[I] += s_dx[wave + int(Q) + 1][I][lane]; });
      });
    }
  }
  if (DX != nullptr) {
    for (int off = lps; off < 64; off <<= 1) {
      static_for<NL>([&](auto I) { dxa[I] += __shfl_xor(dxa[I], off, 64); });
    }
    if (slot == 0 && chan_ok) {
      T* drow = DX + (int64_t)node * P::d_in(a);
      static_for<L + 1>([&](auto I) {
        constexpr int l = I;
        const int off = P::in_off(a, l);
        if (off >= 0) {
          static_for<2 * l + 1>([&](auto M) {
            T* o = &drow[off + u * (2 * l + 1) + M];
            if constexpr (P::kFull) {
              *o = static_cast<T>(dxa[l * l + M]);
            } else {
              *o = (a.acc & 1) ? static_cast<T>(static_cast<A>(*o) + dxa[l * l + M]) : static_cast<T>(dxa[l * l + M]);
            }
          });
        }
      });
    }
  }
}

#if !TPCONV_DD && !TPCONV_DOUBLE
// ------------------------------------------- weights from the radial network
// W = h M, with h [E][H] the edges' hidden features and M [H][P U] the radial
// network's last layer (columns in W's order), generated chunk by chunk on
// the matrix cores into LDS and consumed there, so W never reaches HBM (the
// TrimSO(2) abstract names materialised per-edge tensors as the cost to
// avoid).  One CSR row per block of four wavefronts (eight for U = 64;
// compile-time plans).
// Per chunk of 16 of the row's edges:
//   1. the chunk's h rows go to LDS (zero rows past the row's end);
//   2. v_mfma_f32_16x16x4f32 with M = the 16 edges, N = W's columns, K = H:
//      wavefront w takes the column tiles w, w + 4, ...; K runs in units of
//      16 (step s of unit g uses k = 16 g + 4 kq + s), so a lane's four A
//      values of a unit are one 16-byte LDS read; B (rows of M) comes from
//      L2, the next tile's values in flight while a tile runs; the results
//      fill an LDS tile [edge][column];
//   3. the tensor product of the chunk's edges, the wavefront's slots side
//      by side as in the forward kernel, with the weights read from the tile.
// The backward walks the source-sorted rows the same way: each edge's dW
// overwrites its W in the tile (a lane reads all of its weights before it
// writes any), and then dh = dW M^T runs on the matrix cores (M = edges,
// N = hidden, K = W's columns in units of 16, 16-byte loads of M's rows);
// dW also goes to HBM when asked for (the layer's own gradient
// dM = h^T dW is then a plain product outside).  Row sums are fp64 per lane;
// the wavefronts' sums meet in LDS at the row's end.
typedef float rv4f __attribute__((ext_vector_type(4)));

// M's address, opaque to the compiler at each use: M's values are the same
// for every chunk, and without this the loads of every chunk's products are
// hoisted out of the chunk loop and held in (spilled) registers
__device__ __forceinline__ const float* radial_opaque(const float* p) {
  int z;
  asm volatile("s_mov_b32 %0, 0" : "=s"(z));
  return p + z;
}

__device__ __forceinline__ rv4f rmfma(float a, float b, rv4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

constexpr int kRMaxLgH = 7;  // H = 16 .. 128; the h tile [16][H + 4] is dynamic LDS

template <int L, int U>
struct RShape {
  static constexpr int WS = U * even_count(L);  // W's columns
  static constexpr int SW = WS + 4;             // LDS row stride of the W tile (floats)
  static constexpr int NTILE = WS / 16;
  // wavefronts per block: the W tile of U = 64 fills most of a CU's LDS, so
  // its block has eight wavefronts (two per SIMD) instead of four
  static constexpr int NW = U == 64 ? 8 : 4;
  static constexpr bool kFits = (16 * SW + 16 * ((1 << kRMaxLgH) + 4)) * 4 <= 160 * 1024;
  static_assert(WS % 16 == 0, "W's columns come in tiles of 16");
};

// the chunk's h rows (cn of them) into sH; zero rows after them
__device__ __forceinline__ void radial_stage_h(float* sH, const float* __restrict__ hp, int lgH,
                                               const int32_t* __restrict__ eid, int c0, int cn) {
  const int H = 1 << lgH;
  for (int i = threadIdx.x; i < 16 * H; i += blockDim.x) {
    const int r = i >> lgH, k = i & (H - 1);
    sH[r * (H + 4) + k] = r < cn ? hp[(int64_t)eid[c0 + r] * H + k] : 0.f;
  }
}

// sW[e][c] = sum_k sH[e][k] M[k][c] for this wavefront's column tiles
// (wave, wave + nw, ...)
template <int WS, int SW, int HQ>
__device__ __forceinline__ void radial_gen_w(float* sW, const float* sH, const float* __restrict__ Mw, int wave,
                                             int nw, int lane) {
  constexpr int NTILE = WS / 16;
  Mw = radial_opaque(Mw);
  const int er = lane & 15, kq = lane >> 4;
  rv4f af[HQ];
  static_for<HQ>([&](auto G) {
    af[G] = *reinterpret_cast<const rv4f*>(&sH[er * (16 * HQ + 4) + 16 * int(G) + 4 * kq]);
  });
  auto load_b = [&](int n, float (&b)[4 * HQ]) {
    const float* mc = Mw + 16 * n + er;
    static_for<HQ>([&](auto G) {
      static_for<4>([&](auto S) { b[4 * G + S] = mc[(int64_t)(16 * int(G) + 4 * kq + int(S)) * WS]; });
    });
  };
  // the next tile's B values are loaded once this tile's products are issued
  float b[4 * HQ];
  if (wave < NTILE) load_b(wave, b);
  for (int n = wave; n < NTILE; n += nw) {
    rv4f acc = {0.f, 0.f, 0.f, 0.f};
    static_for<HQ>([&](auto G) {
      static_for<4>([&](auto S) { acc = rmfma(af[G][int(S)], b[4 * G + S], acc); });
    });
    if (n + nw < NTILE) load_b(n + nw, b);
    static_for<4>([&](auto R) { sW[(4 * kq + int(R)) * SW + 16 * n + er] = acc[int(R)]; });
  }
}

template <int WS, int SW>
__device__ __forceinline__ void radial_gen_w_any(float* sW, const float* sH, const float* __restrict__ Mw, int lgH,
                                                 int wave, int nw, int lane) {
  switch (lgH) {
    case 4: radial_gen_w<WS, SW, 1>(sW, sH, Mw, wave, nw, lane); break;
    case 5: radial_gen_w<WS, SW, 2>(sW, sH, Mw, wave, nw, lane); break;
    case 6: radial_gen_w<WS, SW, 4>(sW, sH, Mw, wave, nw, lane); break;
    default: radial_gen_w<WS, SW, 8>(sW, sH, Mw, wave, nw, lane); break;
  }
}

// dh[e][j] = sum_c sW[e][c] M[j][c] for the chunk's cn edges; wavefront w
// takes the hidden tiles w, w + nw, ...
template <int WS, int SW>
__device__ __forceinline__ void radial_gen_dh(const float* sW, const float* __restrict__ Mw,
                                              float* __restrict__ dh, int lgH, const int32_t* __restrict__ eid,
                                              int c0, int cn, int wave, int nw, int lane) {
  const int er = lane & 15, kq = lane >> 4;
  const int H = 1 << lgH;
  Mw = radial_opaque(Mw);
  for (int n = wave; n < (H >> 4); n += nw) {
    rv4f acc = {0.f, 0.f, 0.f, 0.f};
    const float* mrow = Mw + (int64_t)(16 * n + er) * WS + 4 * kq;
    const float* arow = sW + er * SW + 4 * kq;
    // four units of K per trip, the trips kept rolled (a fully unrolled loop
    // reads the whole tile row into registers up front)
    constexpr int NG = WS / 16;
#pragma unroll 1
    for (int g0 = 0; g0 < NG; g0 += 4) {
      static_for<4>([&](auto I) {
        const int g = g0 + int(I);
        if (NG % 4 == 0 || g < NG) {
          const rv4f bv = *reinterpret_cast<const rv4f*>(mrow + 16 * g);
          const rv4f av = *reinterpret_cast<const rv4f*>(arow + 16 * g);
          static_for<4>([&](auto S) { acc = rmfma(av[int(S)], bv[int(S)], acc); });
        }
      });
    }
    static_for<4>([&](auto R) {
      const int r = 4 * kq + int(R);
      if (r < cn) dh[(int64_t)eid[c0 + r] * H + 16 * n + er] = acc[int(R)];
    });
  }
}

// Forward with W = h M: out = the convolution (destination-sorted rows).
template <int L, int U>
__global__ __attribute__((amdgpu_flat_work_group_size(1, 64 * RShape<L, U>::NW))) void rfwd_kernel(const KernelArgs a, const float* __restrict__ hp,
                                                   const float* __restrict__ Mw, int lgH) {
  using P = FullPlan<L, U>;
  using F = Fwd<float, L, P>;
  using S = RShape<L, U>;
  constexpr int NL = F::NL, NT = F::NT;
  constexpr int NSL = 64 >> P::kLg;
  __shared__ __attribute__((aligned(16))) float sW[16 * S::SW];
  extern __shared__ __attribute__((aligned(16))) float sH[];  // [16][H + 4], sized at launch
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int node = a.order[blockIdx.x];
  const int slot = lane >> P::kLg, u = lane & (U - 1);
  const float* __restrict__ X = static_cast<const float*>(a.x);
  const float* __restrict__ Yp = static_cast<const float*>(a.Y);
  const int beg = a.row_ptr[node], end = a.row_ptr[node + 1];
  double rs[NL];
  static_for<NL>([&](auto I) { rs[I] = 0.0; });
  // (Requesting a step's inputs before the products, as the backward does,
  // costs the registers of a third wavefront per SIMD here and measured
  // slower.)
  for (int c0 = beg; c0 < end; c0 += 16) {
    const int cn = min(16, end - c0);
    radial_stage_h(sH, hp, lgH, a.eid, c0, cn);
    __syncthreads();
    radial_gen_w_any<S::WS, S::SW>(sW, sH, Mw, lgH, wave, S::NW, lane);
    __syncthreads();
#pragma unroll 1
    for (int q0 = 0; q0 < cn; q0 += S::NW * NSL) {
      const int q = q0 + wave * NSL + slot;
      if (q < cn) {
        const int e = a.eid[c0 + q], j = a.col[c0 + q];
        float x[NL], y[NL], w[NT];
        const float* xr = X + (int64_t)j * P::kD;
        static_for<L + 1>([&](auto I) {
          constexpr int l = I;
          static_for<2 * l + 1>([&](auto M) { x[l * l + M] = xr[U * l * l + u * (2 * l + 1) + M]; });
        });
        const float* yr = Yp + (int64_t)e * NL;
        static_for<NL>([&](auto I) { y[I] = ldg_stream(yr + I); });
        const float* wr = sW + q * S::SW + u;
        static_for<NT>([&](auto I) {
          if constexpr (P::template on<I>(a)) w[I] = wr[P::template woff<I>(a)];
          else w[I] = 0.f;
        });
        float te[NL];
        F::edge(a, __builtin_amdgcn_readfirstlane(e), x, y, w, te);
        static_for<NL>([&](auto I) { rs[I] += static_cast<double>(te[I]); });
      }
    }
    __syncthreads();  // the next chunk overwrites sH and sW
  }
  // the wavefronts' row sums meet in LDS (over the W tile, or a buffer
  // of its own where the tile is too small), then the slots' by shuffles
  constexpr bool kAlias = 16 * S::SW * 4 >= S::NW * NL * 64 * 8;
  __shared__ double s_red[kAlias ? 1 : S::NW * NL * 64];
  double* red = kAlias ? reinterpret_cast<double*>(sW) : s_red;
  static_for<NL>([&](auto I) { red[(wave * NL + I) * 64 + lane] = rs[I]; });
  __syncthreads();
  if (wave != 0) return;
  static_for<NL>([&](auto I) {
    double t = red[I * 64 + lane];
    static_for<S::NW - 1>([&](auto V) { t += red[((int(V) + 1) * NL + I) * 64 + lane]; });
    rs[I] = t;
  });
  for (int off = U; off < 64; off <<= 1) {
    static_for<NL>([&](auto I) { rs[I] += __shfl_xor(rs[I], off, 64); });
  }
  if (slot == 0) {
    float* orow = static_cast<float*>(a.out) + (int64_t)node * P::kD;
    static_for<L + 1>([&](auto I) {
      constexpr int l = I;
      static_for<2 * l + 1>([&](auto M) { orow[U * l * l + u * (2 * l + 1) + M] = static_cast<float>(rs[l * l + M]); });
    });
  }
}

// Backward with W = h M (source-sorted rows): grad_x (a.out), grad_Y
// (a.dY), dh, and grad_W (a.dW) when not null; each output may be null.
template <int L, int U>
__global__ __attribute__((amdgpu_flat_work_group_size(1, 64 * RShape<L, U>::NW))) void rbwd_kernel(const KernelArgs a, const float* __restrict__ hp,
                                                   const float* __restrict__ Mw, float* __restrict__ dh, int lgH) {
  using P = FullPlan<L, U>;
  using B = Bwd<float, L, P>;
  using S = RShape<L, U>;
  constexpr int NL = B::NL, NT = B::NT;
  constexpr int NV = pow2_ceil(NL);
  constexpr int NSL = 64 >> P::kLg;
  __shared__ __attribute__((aligned(16))) float sW[16 * S::SW];
  extern __shared__ __attribute__((aligned(16))) float sH[];  // [16][H + 4], sized at launch
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int node = a.order[blockIdx.x];
  const int slot = lane >> P::kLg, u = lane & (U - 1);
  const float* __restrict__ Yp = static_cast<const float*>(a.Y);
  const float* __restrict__ Gp = static_cast<const float*>(a.G);
  float* __restrict__ DX = static_cast<float*>(a.out);
  float* __restrict__ DY = static_cast<float*>(a.dY);
  float* __restrict__ DW = static_cast<float*>(a.dW);
  float x[NL];
  {
    const float* xr = static_cast<const float*>(a.x) + (int64_t)node * P::kD;
    static_for<L + 1>([&](auto I) {
      constexpr int l = I;
      static_for<2 * l + 1>([&](auto M) { x[l * l + M] = xr[U * l * l + u * (2 * l + 1) + M]; });
    });
  }
  double dxa[NL];
  static_for<NL>([&](auto I) { dxa[I] = 0.0; });
  const int beg = a.row_ptr[node], end = a.row_ptr[node + 1];
  // A slot past the chunk's end works on the chunk's first edge (valid
  // addresses) and stores nothing, so the dY shuffles stay converged; a
  // wavefront with no edge left skips the step.
  auto load_in = [&](int c0, int q, int& e, float (&g)[NL], float (&y)[NL]) {
    e = a.eid[c0 + q];
    const float* gr = Gp + (int64_t)a.col[c0 + q] * P::kD;
    static_for<L + 1>([&](auto I) {
      constexpr int l = I;
      static_for<2 * l + 1>([&](auto M) { g[l * l + M] = gr[U * l * l + u * (2 * l + 1) + M]; });
    });
    const float* yr = Yp + (int64_t)e * NL;
    static_for<NL>([&](auto I) { y[I] = ldg_stream(yr + I); });
  };
  auto step = [&](int q, bool valid, int e, const float (&g)[NL], const float (&y)[NL]) {
    float w[NT];
    float* wr = sW + q * S::SW + u;
    static_for<NT>([&](auto I) {
      if constexpr (P::template on<I>(a)) w[I] = wr[P::template woff<I>(a)];
      else w[I] = 0.f;
    });
    float dya[NV], dxe[NL];
    static_for<NV>([&](auto I) { dya[I] = 0.f; });
    B::edge(a, __builtin_amdgcn_readfirstlane(e), x, y, g, w, dxe, dya, valid, wr);  // dW over W in the tile
    static_for<NL>([&](auto I) { dxa[I] += valid ? static_cast<double>(dxe[I]) : 0.0; });
    if (DY != nullptr) {
      // reduce-scatter of the NV dY values over the slot's U lanes (as in
      // the backward kernel): lanes with bit b set keep the upper half
      int base = 0, nv = NV;
      static_for<6>([&](auto SS) {
        constexpr int s = SS;
        const int b = U >> (s + 1);
        if (b >= 1) {
          if constexpr ((NV >> s) > 1) {
            constexpr int hh = NV >> (s + 1);
            const bool upper = (u & b) != 0;
            static_for<hh>([&](auto V) {
              float lo = dya[V], hi = dya[V + hh];
              pin_vgpr(lo);
              pin_vgpr(hi);
              const float keep = upper ? hi : lo;
              const float send = upper ? lo : hi;
              dya[V] = keep + __shfl_xor(send, b, 64);
            });
            if (upper) base += hh;
            nv = hh;
          } else {
            dya[0] += __shfl_xor(dya[0], b, 64);
          }
        }
      });
      const int plain_mask = U > NV ? U / NV - 1 : 0;
      if ((u & plain_mask) == 0 && valid) {
        float* dyr = DY + (int64_t)e * NL;
        static_for<NV>([&](auto V) {
          if (V < nv && base + V < NL) dyr[base + V] = dya[V];
        });
      }
    }
  };
  for (int c0 = beg; c0 < end; c0 += 16) {
    const int cn = min(16, end - c0);
    // the first step's inputs are requested before the products
    const bool w0 = wave * NSL < cn;  // wavefront-uniform
    const int q_0 = wave * NSL + slot;
    const bool v_0 = q_0 < cn;
    int e0 = 0;
    float g0[NL], y0[NL];
    if (w0) load_in(c0, v_0 ? q_0 : 0, e0, g0, y0);
    radial_stage_h(sH, hp, lgH, a.eid, c0, cn);
    __syncthreads();
    radial_gen_w_any<S::WS, S::SW>(sW, sH, Mw, lgH, wave, S::NW, lane);
    __syncthreads();
    if (w0) step(v_0 ? q_0 : 0, v_0, e0, g0, y0);
#pragma unroll 1
    for (int q0 = S::NW * NSL; q0 + wave * NSL < cn; q0 += S::NW * NSL) {
      const int q = q0 + wave * NSL + slot;
      const bool valid = q < cn;
      int e;
      float g[NL], y[NL];
      load_in(c0, valid ? q : 0, e, g, y);
      step(valid ? q : 0, valid, e, g, y);
    }
    __syncthreads();  // the chunk's dW is complete in the tile
    if (DW != nullptr) {
      for (int t = threadIdx.x; t < cn * S::WS; t += 64 * S::NW) {
        const int r = t / S::WS, c = t - r * S::WS;
        __builtin_nontemporal_store(sW[r * S::SW + c], DW + (int64_t)a.eid[c0 + r] * S::WS + c);
      }
    }
    if (dh != nullptr) radial_gen_dh<S::WS, S::SW>(sW, Mw, dh, lgH, a.eid, c0, cn, wave, S::NW, lane);
    __syncthreads();  // the next chunk overwrites sH and sW
  }
  if (DX == nullptr) return;  // block-uniform
  constexpr bool kAlias = 16 * S::SW * 4 >= S::NW * NL * 64 * 8;
  __shared__ double s_red[kAlias ? 1 : S::NW * NL * 64];
  double* red = kAlias ? reinterpret_cast<double*>(sW) : s_red;
  static_for<NL>([&](auto I) { red[(wave * NL + I) * 64 + lane] = dxa[I]; });
  __syncthreads();
  if (wave != 0) return;
  static_for<NL>([&](auto I) {
    double t = red[I * 64 + lane];
    static_for<S::NW - 1>([&](auto V) { t += red[((int(V) + 1) * NL + I) * 64 + lane]; });
    dxa[I] = t;
  });
  for (int off = U; off < 64; off <<= 1) {
    static_for<NL>([&](auto I) { dxa[I] += __shfl_xor(dxa[I], off, 64); });
  }
  if (slot == 0) {
    float* drow = DX + (int64_t)node * P::kD;
    static_for<L + 1>([&](auto I) {
      constexpr int l = I;
      static_for<2 * l + 1>([&](auto M) { drow[U * l * l + u * (2 * l + 1) + M] = static_cast<float>(dxa[l * l + M]); });
    });
  }
}

template <int U>
hipError_t launch_radial_u(bool fwd, const KernelArgs& a, const float* h, const float* M, float* dh, int lgH,
                           hipStream_t s) {
  if constexpr (RShape<TPCONV_L, U>::kFits) {
    const size_t lds_h = sizeof(float) * 16 * ((1 << lgH) + 4);
    if (fwd)
      hipLaunchKernelGGL((rfwd_kernel<TPCONV_L, U>), dim3(a.n_rows), dim3(64 * RShape<TPCONV_L, U>::NW), lds_h, s,
                         a, h, M, lgH);
    else
      hipLaunchKernelGGL((rbwd_kernel<TPCONV_L, U>), dim3(a.n_rows), dim3(64 * RShape<TPCONV_L, U>::NW), lds_h, s,
                         a, h, M, dh, lgH);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}
#endif

// ---------------------------------------------------------------- launchers
constexpr bool kDD = TPCONV_DD != 0;

// Graphs with at most this many rows split each row over 4 waves: one wave
// per row would leave most SIMDs with a single wavefront and nothing to hide
// its memory latency behind.
constexpr int kSplitRows = 1024;

template <typename T, class P, int R = 1, int YS = kYGlobal>
hipError_t launch_fwd(const KernelArgs& a, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  const int rows_per_block = 4 / R;
  const int blocks = (a.n_rows + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL((fwd_kernel<T, TPCONV_L, P, kDD, R, YS>), dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, class P, int R = 1, int YS = kYGlobal>
hipError_t launch_bwd(const KernelArgs& a, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  const int rows_per_block = 4 / R;
  const int blocks = (a.n_rows + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL((bwd_kernel<T, TPCONV_L, P, kDD, R, YS>), dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

bool all_even(const KernelArgs& a) {
  constexpr int L = TPCONV_L;
  bool even = true;
  int t = 0;
  for (int l1 = 0; l1 <= L; ++l1)
    for (int l2 = 0; l2 <= L; ++l2)
      for (int l3 = 0; l3 <= L; ++l3)
        if (cg::triangle(l1, l2, l3)) {
          const bool on = t < 64 ? ((a.pmask_lo >> t) & 1ull) : ((a.pmask_hi >> (t - 64)) & 1ull);
          if (on && (l1 + l2 + l3) % 2) even = false;
          ++t;
        }
  return even;
}

// multiplicities with a compile-time kernel for full plans
template <int... Us>
struct UList {};
using FullMuls = UList<16, 32, 64>;

template <typename T, bool FWD, int YS, class FP>
hipError_t launch_full_rows(const KernelArgs& a, hipStream_t s) {
  // the fp64 l = 4 backward with harmonics from vectors holds ~117 KB of LDS
  // per block: no room for the split rows' LDS as well
  constexpr bool kWhole = YS == kYVec && !FWD && sizeof(T) == 8 && TPCONV_L >= 4;
  if constexpr (FWD) {
    if (a.n_rows <= kSplitRows) return launch_fwd<T, FP, 4, YS>(a, s);
    return launch_fwd<T, FP, 1, YS>(a, s);
  } else {
    if constexpr (!kWhole) {
      if (a.n_rows <= kSplitRows) return launch_bwd<T, FP, 4, YS>(a, s);
    }
    return launch_bwd<T, FP, 1, YS>(a, s);
  }
}


template <typename T, bool FWD, int U0, int... Us>
bool launch_full(const KernelArgs& a, hipStream_t s, hipError_t& err, UList<U0, Us...>) {
  if (a.mul == U0) {
    using FP = FullPlan<TPCONV_L, U0>;
    if constexpr (!kDD) {
      if constexpr (FWD && sizeof(T) == 8 && TPCONV_L == 4) {
        if (a.from_vec) {  // the same split with the harmonics evaluated in each launch
          err = launch_full_rows<T, true, kYVec, FullPlanPart<4, U0, 0b10011>>(a, s);
          if (err == hipSuccess) err = launch_full_rows<T, true, kYVec, FullPlanPart<4, U0, 0b01100>>(a, s);
          return true;
        }
      }
      if (a.from_vec) {
        err = launch_full_rows<T, FWD, kYVec, FP>(a, s);
        return true;
      }
      if constexpr (FWD && sizeof(T) == 8 && TPCONV_L == 4) {
        // fp64, l <= 4: output l's {0, 1, 4} and {2, 3} in two launches (one
        // launch needs 256 VGPRs + ~100 AGPRs, one wavefront per SIMD; each
        // part fits 221-239 VGPRs, two wavefronts per SIMD; c2k forward
        // 0.221 -> 0.206 ms)
        err = launch_full_rows<T, true, kYRows, FullPlanPart<4, U0, 0b10011>>(a, s);
        if (err == hipSuccess) err = launch_full_rows<T, true, kYRows, FullPlanPart<4, U0, 0b01100>>(a, s);
        return true;
      }
      err = launch_full_rows<T, FWD, FWD ? kYRows : kYGlobal, FP>(a, s);
      return true;
    }
    err = launch_full_rows<T, FWD, kYGlobal, FP>(a, s);
    return true;
  }
  if constexpr (sizeof...(Us) > 0) {
    return launch_full<T, FWD, Us...>(a, s, err, UList<Us...>{});
  } else {
    return false;
  }
}

template <typename T, bool FWD, int YS>
hipError_t dispatch_rt(const KernelArgs& a, hipStream_t s) {
  using PE = RtPlan<TPCONV_L, kEvenOnly>;
  using PA = RtPlan<TPCONV_L, kAnyParity>;
  if (all_even(a)) return FWD ? launch_fwd<T, PE, 1, YS>(a, s) : launch_bwd<T, PE, 1, YS>(a, s);
  return FWD ? launch_fwd<T, PA, 1, YS>(a, s) : launch_bwd<T, PA, 1, YS>(a, s);
}

template <typename T, bool FWD>
hipError_t dispatch(const KernelArgs& a, hipStream_t s) {
  hipError_t err = hipSuccess;
  if (a.full_plan && launch_full<T, FWD>(a, s, err, FullMuls{})) return err;
  if constexpr (!kDD) {
    if (a.from_vec) return dispatch_rt<T, FWD, kYVec>(a, s);
  }
  return dispatch_rt<T, FWD, kYGlobal>(a, s);
}

}  // namespace

#define TPCONV_CAT2(a, b) a##b
#define TPCONV_CAT(a, b) TPCONV_CAT2(a, b)
#define TPCONV_LNAME(stem, ty) TPCONV_CAT(TPCONV_CAT(stem, TPCONV_L), ty)

#if TPCONV_DD
#if TPCONV_DOUBLE
hipError_t TPCONV_LNAME(launch_ddf_l, _f64)(const KernelArgs& a, hipStream_t s) { return dispatch<double, true>(a, s); }
hipError_t TPCONV_LNAME(launch_ddb_l, _f64)(const KernelArgs& a, hipStream_t s) { return dispatch<double, false>(a, s); }
#else
hipError_t TPCONV_LNAME(launch_ddf_l, _f32)(const KernelArgs& a, hipStream_t s) { return dispatch<float, true>(a, s); }
hipError_t TPCONV_LNAME(launch_ddb_l, _f32)(const KernelArgs& a, hipStream_t s) { return dispatch<float, false>(a, s); }
#endif
#else
#if TPCONV_DOUBLE
hipError_t TPCONV_LNAME(launch_fwd_l, _f64)(const KernelArgs& a, hipStream_t s) { return dispatch<double, true>(a, s); }
hipError_t TPCONV_LNAME(launch_bwd_l, _f64)(const KernelArgs& a, hipStream_t s) { return dispatch<double, false>(a, s); }
#else
hipError_t TPCONV_LNAME(launch_fwd_l, _f32)(const KernelArgs& a, hipStream_t s) { return dispatch<float, true>(a, s); }
hipError_t TPCONV_LNAME(launch_bwd_l, _f32)(const KernelArgs& a, hipStream_t s) { return dispatch<float, false>(a, s); }
hipError_t TPCONV_LNAME(launch_radial_l, _f32)(bool fwd, const KernelArgs& a, const float* h, const float* M,
                                                float* dh, int lgH, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  if (!a.full_plan || lgH < 4 || lgH > kRMaxLgH) return hipErrorInvalidValue;
  switch (a.mul) {
    case 16: return launch_radial_u<16>(fwd, a, h, M, dh, lgH, s);
    case 32: return launch_radial_u<32>(fwd, a, h, M, dh, lgH, s);
    case 64: return launch_radial_u<64>(fwd, a, h, M, dh, lgH, s);
    default: return hipErrorInvalidValue;
  }
}
#endif
#endif

}  // namespace tpconv
