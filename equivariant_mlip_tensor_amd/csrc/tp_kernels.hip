// tp_kernels.hip -- fused CGTP convolution kernels for gfx950 (CDNA4).
//
// Compiled once per l bound (-DTPCONV_L=0..4); each object defines the four
// launchers declared in tp_common.hpp for that bound.
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
#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>

#include "tp_common.hpp"

#ifndef TPCONV_L
#error "compile with -DTPCONV_L=<l bound>"
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

// Path parity classes a kernel is specialised for.
enum Parity { kAnyParity = 0, kEvenOnly = 1 };

constexpr bool triple_in_class(int l1, int l2, int l3, int par) {
  return par == kAnyParity || ((l1 + l2 + l3) % 2 == 0);
}

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

template <int T>
__device__ __forceinline__ bool present(const KernelArgs& a) {
  if constexpr (T < 64)
    return (a.pmask_lo >> T) & 1ull;
  else
    return (a.pmask_hi >> (T - 64)) & 1ull;
}

template <int T>
__device__ __forceinline__ bool first3(const KernelArgs& a) {
  if constexpr (T < 64)
    return (a.first3_lo >> T) & 1ull;
  else
    return (a.first3_hi >> (T - 64)) & 1ull;
}

template <int T>
__device__ __forceinline__ bool first1(const KernelArgs& a) {
  if constexpr (T < 64)
    return (a.first1_lo >> T) & 1ull;
  else
    return (a.first1_hi >> (T - 64)) & 1ull;
}

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

template <int L, int PAR, int L1, int L2>
__device__ __forceinline__ bool group_present(const KernelArgs& a) {
  bool any = false;
  static_for<L + 1>([&](auto I3) {
    constexpr int l3 = I3;
    if constexpr (cg::triangle(L1, L2, l3) && triple_in_class(L1, L2, l3, PAR))
      any = any || present<triple_id(L, L1, L2, l3)>(a);
  });
  return any;
}

template <typename T>
__device__ __forceinline__ T ldg_stream(const T* p) {
  return __builtin_nontemporal_load(p);
}

// ------------------------------------------------------------------ forward
template <typename T, int L, int PAR>
struct Fwd {
  static constexpr int NL = (L + 1) * (L + 1);
  static constexpr int NT = triple_count(L);

  // te[l3 block] = sum over the edge's paths into l3 of W[p,u] * CG_p(x, y)
  static __device__ __forceinline__ void edge(const KernelArgs& a, const T (&x)[NL], const T (&y)[NL],
                                              const T (&w)[NT], T (&te)[NL]) {
    static_for<L + 1>([&](auto I1) {
      constexpr int l1 = I1;
      static_for<L + 1>([&](auto I2) {
        constexpr int l2 = I2;
        if (!group_present<L, PAR, l1, l2>(a)) return;
        constexpr int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1;
        T pr[n1 * n2];
        static_for<n1>([&](auto M1) {
          static_for<n2>([&](auto M2) {
            if constexpr (group_uses<L, PAR, l1, l2>(M1, M2)) pr[M1 * n2 + M2] = x[l1 * l1 + M1] * y[l2 * l2 + M2];
          });
        });
        static_for<L + 1>([&](auto I3) {
          constexpr int l3 = I3;
          if constexpr (cg::triangle(l1, l2, l3) && triple_in_class(l1, l2, l3, PAR)) {
            constexpr int t = triple_id(L, l1, l2, l3);
            if (present<t>(a)) {
              using TI = TabInfo<l1, l2, l3>;
              constexpr int n3 = 2 * l3 + 1;
              T z[n3];
              static_for<TI::tab.n>([&](auto K) {
                constexpr cg::Entry en = TI::tab.e[K];
                constexpr T c = en.neg ? T(-en.mag) : T(en.mag);
                const T p = pr[en.m1 * n2 + en.m2];
                if constexpr (TI::first_m3(K))
                  z[en.m3] = c * p;
                else
                  z[en.m3] = fmaT(c, p, z[en.m3]);
              });
              if (first3<t>(a)) {
                static_for<n3>([&](auto M3) { te[l3 * l3 + M3] = w[t] * z[M3]; });
              } else {
                static_for<n3>([&](auto M3) { te[l3 * l3 + M3] = fmaT(w[t], z[M3], te[l3 * l3 + M3]); });
              }
            }
          }
        });
      });
    });
  }
};

template <typename T, int L, int PAR>
__global__ __launch_bounds__(256) void fwd_kernel(const KernelArgs a) {
  using F = Fwd<T, L, PAR>;
  constexpr int NL = F::NL, NT = F::NT;
  const int lane = threadIdx.x & 63;
  const int node = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (node >= a.n_rows) return;  // wave-uniform
  const int slot = lane >> a.lps_log2;
  const int u = lane & ((1 << a.lps_log2) - 1);
  const bool chan_ok = u < a.mul;
  const int uc = chan_ok ? u : 0;  // inactive lanes read channel 0 (valid addresses), never store

  const T* __restrict__ X = static_cast<const T*>(a.x);
  const T* __restrict__ Yp = static_cast<const T*>(a.Y);
  const T* __restrict__ Wp = static_cast<const T*>(a.W);
  T* __restrict__ O = static_cast<T*>(a.out);

  using A = typename RowAcc<T>::type;
  A acc[NL];
  static_for<NL>([&](auto I) { acc[I] = A(0); });

  const int beg = a.row_ptr[node];
  const int end = a.row_ptr[node + 1];
  for (int k = beg + slot; k < end; k += a.nslots) {
    const int e = a.eid[k];
    const int j = a.col[k];
    T x[NL], y[NL], w[NT];
    const T* xr = X + (int64_t)j * a.d_in;
    static_for<L + 1>([&](auto I) {
      constexpr int l = I;
      const int off = a.in_off[l];
      static_for<2 * l + 1>([&](auto M) {
        x[l * l + M] = off >= 0 ? xr[off + uc * (2 * l + 1) + M] : T(0);
      });
    });
    const T* yr = Yp + (int64_t)e * a.d_sh;
    static_for<NL>([&](auto I) {
      if (I < a.d_sh) y[I] = ldg_stream(yr + I);
      else y[I] = T(0);
    });
    const T* wr = Wp + (int64_t)e * a.wstride + uc;
    static_for<NT>([&](auto I) {
      if (present<I>(a)) w[I] = ldg_stream(wr + a.woff[I]);
      else w[I] = T(0);
    });
    T te[NL];
    F::edge(a, x, y, w, te);
    static_for<L + 1>([&](auto I) {
      constexpr int l = I;
      if ((a.out_l_mask >> l) & 1) {
        static_for<2 * l + 1>([&](auto M) { acc[l * l + M] += static_cast<A>(te[l * l + M]); });
      }
    });
  }

  // sum the slots' partial rows: slots sit at lane offsets 2^lps_log2 .. 32
  for (int off = 1 << a.lps_log2; off < 64; off <<= 1) {
    static_for<NL>([&](auto I) { acc[I] += __shfl_xor(acc[I], off, 64); });
  }
  if (slot == 0 && chan_ok) {
    T* orow = O + (int64_t)node * a.d_out;
    static_for<L + 1>([&](auto I) {
      constexpr int l = I;
      const int off = a.out_off[l];
      if (off >= 0) {
        static_for<2 * l + 1>([&](auto M) { orow[off + u * (2 * l + 1) + M] = static_cast<T>(acc[l * l + M]); });
      }
    });
  }
}

// ----------------------------------------------------------------- backward
template <typename T, int L, int PAR>
struct Bwd {
  static constexpr int NL = (L + 1) * (L + 1);
  static constexpr int NT = triple_count(L);

  // One edge: dW for every path (unreduced), and per-lane contributions to dx
  // (accumulated over the row) and to dY (summed over channels afterwards).
  template <int NV>
  static __device__ __forceinline__ void edge(const KernelArgs& a, const T (&x)[NL], const T (&y)[NL],
                                              const T (&g)[NL], const T (&w)[NT], T (&dxe)[NL],
                                              T (&dya)[NV], T (&dw)[NT]) {
    static_assert(NV >= NL, "dY accumulator too short");
    static_for<L + 1>([&](auto I1) {
      constexpr int l1 = I1;
      static_for<L + 1>([&](auto I2) {
        constexpr int l2 = I2;
        static_for<L + 1>([&](auto I3) {
          constexpr int l3 = I3;
          if constexpr (cg::triangle(l1, l2, l3) && triple_in_class(l1, l2, l3, PAR)) {
            constexpr int t = triple_id(L, l1, l2, l3);
            if (present<t>(a)) {
              using TI = TabInfo<l1, l2, l3>;
              constexpr int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1;
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
              dw[t] = s;
              if (first1<t>(a)) {
                static_for<n1>([&](auto M1) {
                  if constexpr (TI::has_m1(M1)) dxe[l1 * l1 + M1] = w[t] * dxp[M1];
                  else dxe[l1 * l1 + M1] = T(0);
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

constexpr int pow2_ceil(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

template <typename T, int L, int PAR>
__global__ __launch_bounds__(256) void bwd_kernel(const KernelArgs a) {
  using B = Bwd<T, L, PAR>;
  constexpr int NL = B::NL, NT = B::NT;
  constexpr int NV = pow2_ceil(NL);  // dY values, padded to a power of two for the reduce-scatter
  const int lane = threadIdx.x & 63;
  const int node = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (node >= a.n_rows) return;  // wave-uniform
  const int lps = 1 << a.lps_log2;
  const int slot = lane >> a.lps_log2;
  const int u = lane & (lps - 1);
  const bool chan_ok = u < a.mul;
  const int uc = chan_ok ? u : 0;

  const T* __restrict__ X = static_cast<const T*>(a.x);
  const T* __restrict__ Yp = static_cast<const T*>(a.Y);
  const T* __restrict__ Wp = static_cast<const T*>(a.W);
  const T* __restrict__ Gp = static_cast<const T*>(a.G);
  T* __restrict__ DX = static_cast<T*>(a.out);
  T* __restrict__ DY = static_cast<T*>(a.dY);
  T* __restrict__ DW = static_cast<T*>(a.dW);

  // this source node's features stay in registers for the whole row; lanes
  // beyond U hold zeros so they add nothing to the channel sums of dY
  T x[NL];
  {
    const T* xr = X + (int64_t)node * a.d_in;
    static_for<L + 1>([&](auto I) {
      constexpr int l = I;
      const int off = a.in_off[l];
      static_for<2 * l + 1>([&](auto M) {
        x[l * l + M] = (off >= 0 && chan_ok) ? xr[off + u * (2 * l + 1) + M] : T(0);
      });
    });
  }
  using A = typename RowAcc<T>::type;
  A dxa[NL];
  static_for<NL>([&](auto I) { dxa[I] = A(0); });

  const int beg = a.row_ptr[node];
  const int end = a.row_ptr[node + 1];
  for (int k = beg + slot; k < end; k += a.nslots) {
    const int e = a.eid[k];
    const int i = a.col[k];
    T g[NL], y[NL], w[NT];
    const T* gr = Gp + (int64_t)i * a.d_out;
    static_for<L + 1>([&](auto I) {
      constexpr int l = I;
      const int off = a.out_off[l];
      static_for<2 * l + 1>([&](auto M) {
        g[l * l + M] = off >= 0 ? gr[off + uc * (2 * l + 1) + M] : T(0);
      });
    });
    const T* yr = Yp + (int64_t)e * a.d_sh;
    static_for<NL>([&](auto I) {
      if (I < a.d_sh) y[I] = ldg_stream(yr + I);
      else y[I] = T(0);
    });
    const T* wr = Wp + (int64_t)e * a.wstride + uc;
    static_for<NT>([&](auto I) {
      if (present<I>(a)) w[I] = ldg_stream(wr + a.woff[I]);
      else w[I] = T(0);
    });

    T dya[NV], dw[NT];
    static_for<NV>([&](auto I) { dya[I] = T(0); });
    T dxe[NL];
    B::edge(a, x, y, g, w, dxe, dya, dw);
    static_for<L + 1>([&](auto I) {
      constexpr int l = I;
      if ((a.in_l_mask >> l) & 1) {
        static_for<2 * l + 1>([&](auto M) { dxa[l * l + M] += static_cast<A>(dxe[l * l + M]); });
      }
    });

    if (DW != nullptr && chan_ok) {
      T* dwr = DW + (int64_t)e * a.wstride + u;
      static_for<NT>([&](auto I) {
        if (present<I>(a)) __builtin_nontemporal_store(dw[I], dwr + a.woff[I]);
      });
    }
    if (DY != nullptr) {
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
              const T keep = upper ? dya[V + h] : dya[V];
              const T send = upper ? dya[V] : dya[V + h];
              dya[V] = keep + __shfl_xor(send, b, 64);
            });
            if (upper) base += h;
            nv = h;
          } else {
            dya[0] += __shfl_xor(dya[0], b, 64);
          }
        }
      });
      // bits below lps/NV were plain sums: one lane of each such group stores
      const int plain_mask = lps > NV ? lps / NV - 1 : 0;
      if ((u & plain_mask) == 0) {
        T* dyr = DY + (int64_t)e * a.d_sh;
        static_for<NV>([&](auto V) {
          if (V < nv && base + V < a.d_sh) dyr[base + V] = dya[V];
        });
      }
    }
  }

  if (DX != nullptr) {
    for (int off = lps; off < 64; off <<= 1) {
      static_for<NL>([&](auto I) { dxa[I] += __shfl_xor(dxa[I], off, 64); });
    }
    if (slot == 0 && chan_ok) {
      T* drow = DX + (int64_t)node * a.d_in;
      static_for<L + 1>([&](auto I) {
        constexpr int l = I;
        const int off = a.in_off[l];
        if (off >= 0) {
          static_for<2 * l + 1>([&](auto M) { drow[off + u * (2 * l + 1) + M] = static_cast<T>(dxa[l * l + M]); });
        }
      });
    }
  }
}

template <typename T, int PAR>
hipError_t launch_fwd(const KernelArgs& a, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  const int waves_per_block = 4;
  const int blocks = (a.n_rows + waves_per_block - 1) / waves_per_block;
  hipLaunchKernelGGL((fwd_kernel<T, TPCONV_L, PAR>), dim3(blocks), dim3(64 * waves_per_block), 0, s, a);
  return hipGetLastError();
}

template <typename T, int PAR>
hipError_t launch_bwd(const KernelArgs& a, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  const int waves_per_block = 4;
  const int blocks = (a.n_rows + waves_per_block - 1) / waves_per_block;
  hipLaunchKernelGGL((bwd_kernel<T, TPCONV_L, PAR>), dim3(blocks), dim3(64 * waves_per_block), 0, s, a);
  return hipGetLastError();
}

bool all_even(const KernelArgs& a) {
  constexpr int L = TPCONV_L;
  bool even = true;
  int t = 0;
  for (int l1 = 0; l1 <= L; ++l1)
    for (int l2 = 0; l2 <= L; ++l2)
      for (int l3 = 0; l3<= L; ++l3)
        if (cg::triangle(l1, l2, l3)) {
          const bool on = t < 64 ? ((a.pmask_lo >> t) & 1ull) : ((a.pmask_hi >> (t - 64)) & 1ull);
          if (on && (l1 + l2 + l3) % 2) even = false;
          ++t;
        }
  return even;
}

}  // namespace

#define TPCONV_CAT2(a, b) a##b
#define TPCONV_CAT(a, b) TPCONV_CAT2(a, b)
#define TPCONV_LNAME(stem, ty) TPCONV_CAT(TPCONV_CAT(stem, TPCONV_L), ty)

hipError_t TPCONV_LNAME(launch_fwd_l, _f32)(const KernelArgs& a, hipStream_t s) {
  return all_even(a) ? launch_fwd<float, kEvenOnly>(a, s) : launch_fwd<float, kAnyParity>(a, s);
}
hipError_t TPCONV_LNAME(launch_fwd_l, _f64)(const KernelArgs& a, hipStream_t s) {
  return all_even(a) ? launch_fwd<double, kEvenOnly>(a, s) : launch_fwd<double, kAnyParity>(a, s);
}
hipError_t TPCONV_LNAME(launch_bwd_l, _f32)(const KernelArgs& a, hipStream_t s) {
  return all_even(a) ? launch_bwd<float, kEvenOnly>(a, s) : launch_bwd<float, kAnyParity>(a, s);
}
hipError_t TPCONV_LNAME(launch_bwd_l, _f64)(const KernelArgs& a, hipStream_t s) {
  return all_even(a) ? launch_bwd<double, kEvenOnly>(a, s) : launch_bwd<double, kAnyParity>(a, s);
}

}  // namespace tpconv
