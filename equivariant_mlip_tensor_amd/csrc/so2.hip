// so2.hip -- SO(2) convolution on gfx950 (fp32).
//
// The operation (TrimSO(2), Abstract: rotation on gather, dense matrix
// multiplications in the edge frame, inverse rotation on reduction), per edge
// e with neighbour j and centre i:
//   x~[l][c][m]  = sum_n D_e^l[m][n] x[j][l][c][n]          (rotation on gather)
//   m = 0:  y~_0  = A_0 X_0
//   m > 0:  y~_+m = A_m X_+m - B_m X_-m,  y~_-m = B_m X_+m + A_m X_-m
//           (X_+-m: x~[l][c][+-m] over l = m..L, c, index (l - m) C + c)
//   out[i][l][c][n] += sum_m D_e^l[m][n] y~[l][c][m]      (inverse rotation on reduction)
// with A_m, B_m shared by all edges.  The backward needs grad_x, which is the
// same operator with the adjoint maps (A^T, and B^T with the opposite sign)
// run over the source-sorted rows on grad_out, and the map gradients, sums
// over all edges of outer products of the rotated grad_out and x.
//
// Kernels (one wavefront = 64 lanes):
//  * k_so2_conv<L, C, ADJ>: one CSR row per block of two wavefronts, edges
//    in chunks of 16.  Per chunk: the 16 Wigner rows go to LDS; each
//    wavefront rotates 8 neighbour rows in registers (lane = channel c and a
//    share of the m) into an LDS tile [edge][node layout]; per |m| the maps
//    run on the matrix cores (v_mfma_f32_16x16x4f32: M = the 16 edges,
//    N = output (l, c), K = input (l, c)), the wavefronts splitting the
//    n-tiles, A and B fragments shared by the four products of a (+m, -m)
//    pair, weights streamed from L2 a unit ahead; after a barrier the
//    results overwrite the tile at the same (+-m) places; the inverse
//    rotation then adds each edge's message into per-lane row sums, which
//    the two wavefronts combine once per row.  Nothing per edge reaches HBM.
//    In the frame-gradient mode (FRAMES) the inverse rotation is replaced by
//    a contraction of the tile (y~, or dx~ for the adjoint) with the row's
//    own vector over channels: the two terms of the gradient with respect to
//    each edge's Wigner blocks, recomputed rather than kept per edge.
//  * k_so2_wgrad<L, C>: eight wavefronts share one LDS copy of the rotated x
//    and grad_out of 16 edges; each wavefront owns a fixed set of 16 x 16
//    output tiles of the map gradients (compile-time list, its accumulators
//    stay in registers over all of the block's edges) and runs them on the
//    matrix cores with K = edges.  Per-block partial sums go to a caller
//    workspace; k_so2_wsum adds them in block order (deterministic, no
//    atomics).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <type_traits>
#include <utility>

#include "tp_common.hpp"

namespace tpconv {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

template <typename F, int... I>
__device__ __forceinline__ void so2_sf(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void so2_for(F&& f) {
  if constexpr (N > 0) so2_sf(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ v4f mfma(float a, float b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int L, int C>
struct So2Shape {
  static_assert(C == 16 || C == 32, "channels: 16 or 32");
  static constexpr int NC = (L + 1) * (L + 1);
  static constexpr int DN = C * NC;                        // node row, floats
  static constexpr int NSPLIT = 64 / C;                    // lanes per channel
  // LDS tile edge strides: 2 mod 32 in the convolution (fragment rows are
  // edges), 16 mod 32 in the map gradient (fragment rows are (l, c), and the
  // two quarter-waves of a half-wave read edges e and e + 1: disjoint banks)
  static constexpr int PAD = (DN + 31) / 32 * 32 + 2;
  static constexpr int PADW = (DN + 31) / 32 * 32 + 16;
  static constexpr int ND = (L + 1) * (2 * L + 1) * (2 * L + 3) / 3;  // Wigner floats per edge
  static constexpr int NDP = ND + 1;                       // LDS stride of a Wigner row
  static constexpr int kEdges = 16;
  static constexpr int K(int m) { return (L + 1 - m) * C; }
  static constexpr int doff(int l) { return l * (2 * l - 1) * (2 * l + 1) / 3; }
  static constexpr int xoff(int l) { return C * l * l; }
  static constexpr int woffA(int m) {
    int o = 0;
    for (int k = 0; k < m; ++k) o += (k ? 2 : 1) * K(k) * K(k);
    return o;
  }
  static constexpr int woffB(int m) { return woffA(m) + K(m) * K(m); }
  static constexpr int NW = woffA(L + 1);
  static constexpr int J(int l) { return (2 * l + 1 + NSPLIT - 1) / NSPLIT; }  // components per lane, degree l
  static constexpr int jbase(int l) {
    int b = 0;
    for (int k = 0; k < l; ++k) b += J(k);
    return b;
  }
  static constexpr int NACC = jbase(L + 1);
  // map-gradient jobs: one 16 x 16 tile (m, ot, it) of A_m (and of B_m when m > 0)
  static constexpr int njobs() {
    int n = 0;
    for (int m = 0; m <= L; ++m) n += (K(m) / 16) * (K(m) / 16);
    return n;
  }
  struct Job {
    int m, ot, it;
  };
  static constexpr Job job(int j) {
    for (int m = 0; m <= L; ++m) {
      const int t = K(m) / 16;
      if (j < t * t) return Job{m, j / t, j % t};
      j -= t * t;
    }
    return Job{-1, 0, 0};
  }
  // the map-gradient block's wavefronts and their jobs: longest first, each
  // to the least-loaded wavefront (a job costs 4 products per k-step when
  // m > 0, one when m = 0)
  static constexpr int kWaves = 8;
  struct Assign {
    int nmine[kWaves];
    int list[kWaves][njobs()];
  };
  static constexpr Assign assign() {
    Assign a{};
    int load[kWaves] = {};
    for (int pass = 0; pass < 2; ++pass)
      for (int j = 0; j < njobs(); ++j) {
        const bool heavy = job(j).m > 0;
        if (heavy != (pass == 0)) continue;
        int best = 0;
        for (int w = 1; w < kWaves; ++w)
          if (load[w] < load[best]) best = w;
        load[best] += heavy ? 4 : 1;
        a.list[best][a.nmine[best]++] = j;
      }
    return a;
  }
};

template <int L, int C>
struct So2Jobs {
  static constexpr typename So2Shape<L, C>::Assign value = So2Shape<L, C>::assign();
};

// Channel c of a node row: its (L+1)^2 components, (l, n) at l*l + l + n.
template <int L, int C>
__device__ __forceinline__ void load_channel(const float* __restrict__ xr, int c, float (&xv)[(L + 1) * (L + 1)]) {
  using S = So2Shape<L, C>;
  so2_for<L + 1>([&](auto IL) {
    constexpr int l = IL, n2 = 2 * l + 1;
    so2_for<n2>([&](auto N) { xv[l * l + N] = xr[S::xoff(l) + c * n2 + N]; });
  });
}

// Rotates one edge's channel into the tile (rotation on gather): lane (c, h)
// writes x~[l][c][m] for m = h, h + NSPLIT, ...
template <int L, int C>
__device__ __forceinline__ void rotate_in(const float (&xv)[(L + 1) * (L + 1)], const float* dle, float* te, int c,
                                          int h) {
  using S = So2Shape<L, C>;
  so2_for<L + 1>([&](auto IL) {
    constexpr int l = IL, n2 = 2 * l + 1;
    so2_for<S::J(l)>([&](auto JJ) {
      const int m = h + S::NSPLIT * int(JJ);
      if (m < n2) {
        const float* dr = dle + S::doff(l) + m * n2;
        float s = 0.f;
        so2_for<n2>([&](auto N) { s = fmaf(dr[N], xv[l * l + N], s); });
        te[S::xoff(l) + c * n2 + m] = s;
      }
    });
  });
}

// The Wigner rows of a chunk's edges into LDS (zeros past the chunk's end, so
// those edges rotate to zero).  my_id: edge id of chunk edge (lane & 15)
// (any value for lanes past ne); NTH threads share the copy.
template <int L, int C, int NTH>
__device__ __forceinline__ void load_wigner(int tid, int ne, int my_id, const float* __restrict__ Dm, float* dl) {
  using S = So2Shape<L, C>;
  constexpr int TOT = S::kEdges * S::ND, IT = (TOT + NTH - 1) / NTH;
  float v[IT];
  so2_for<IT>([&](auto I) {
    const int q = tid + NTH * int(I);
    const int e = q / S::ND, r = q - e * S::ND;
    const int id = __shfl(my_id, e & 15);
    v[I] = (q < TOT && e < ne) ? Dm[(int64_t)id * S::ND + r] : 0.f;
  });
  so2_for<IT>([&](auto I) {
    const int q = tid + NTH * int(I);
    const int e = q / S::ND, r = q - e * S::ND;
    if (q < TOT) dl[e * S::NDP + r] = v[I];
  });
}

// K index supplied by lane quarter kq at step s of 16-wide unit g.  Any
// permutation of K serves (it applies to both fragments); this one keeps a
// lane's four steps contiguous (one 16-byte weight load).  (Placing the two
// quarters of a half-wave 16 channels apart removes the remaining 2-way LDS
// bank conflicts of the A fragments but costs registers: measured slower.)
template <int C>
__device__ __forceinline__ int so2_k(int g, int kq, int s) {
  return 16 * g + 4 * kq + s;
}

// The per-|m| maps of one chunk on the matrix cores (v_mfma_f32_16x16x4f32:
// M = the 16 edges, N = output (l, c), K = input (l, c)) for the n-tiles
// T = WV, WV + 2, ... of each |m|; the block's other wavefront takes the rest.
// Per |m|: products, a barrier (both wavefronts have read X_+-m), then the
// results overwrite the tile at the same (+-m) places.
template <int L, int C, bool ADJ, int WV>
__device__ __forceinline__ void so2_maps(float* tile, const float* __restrict__ W, const int lane) {
  using S = So2Shape<L, C>;
  const int er = lane & 15;  // A fragment: edge row; B fragment and result: column
  const int kq = lane >> 4;  // A/B fragment: k within the step; result: rows 4 kq .. 4 kq + 3
  so2_for<L + 1>([&](auto IM) {
    constexpr int m = IM;
    constexpr int K = S::K(m), NT = K / 16, NTW = (NT - WV + 1) / 2;
    constexpr int NA = NTW > 0 ? NTW : 1, NB = (m > 0 && NTW > 0) ? NTW : 1;
    const float* WA = W + S::woffA(m);
    const float* WB = W + (m > 0 ? S::woffB(m) : 0);
    v4f yp[NA], ym[NB];
    if constexpr (NTW > 0) {
      so2_for<NTW>([&](auto I) {
        yp[I] = v4f{0.f, 0.f, 0.f, 0.f};
        if constexpr (m > 0) ym[I] = v4f{0.f, 0.f, 0.f, 0.f};
      });
      // K runs in units of 16 (so2_k): a lane's four weights of a unit for
      // one n-tile are W[n][k..k+3], one 16-byte load.  The adjoint gets the
      // maps transposed (k_so2_transpose) and reads them the same way.  The
      // next unit's weights are in flight while this unit's products run.
      constexpr int NG = K / 16;
      auto load_w = [&](const int g, v4f (&wa)[NA], v4f (&wb)[NB]) {
        const int k = so2_k<C>(g, kq, 0);
        so2_for<NTW>([&](auto I) {
          const int n = (WV + 2 * int(I)) * 16 + er;
          wa[I] = *reinterpret_cast<const v4f*>(WA + n * K + k);
          if constexpr (m > 0) wb[I] = *reinterpret_cast<const v4f*>(WB + n * K + k);
        });
      };
      auto run_group = [&](const int g, const v4f (&wa)[NA], const v4f (&wb)[NB]) {
        so2_for<4>([&](auto SS) {
          const int k = so2_k<C>(g, kq, int(SS));
          const int l1 = m + k / C, c1 = k % C;
          const float* t1 = &tile[er * S::PAD + C * l1 * l1 + c1 * (2 * l1 + 1) + l1];
          const float ap = t1[m];
          const float am = m > 0 ? t1[-m] : 0.f;
          so2_for<NTW>([&](auto I) {
            const float a_w = wa[I][int(SS)];
            yp[I] = mfma(ap, a_w, yp[I]);
            if constexpr (m > 0) {
              const float b_w = wb[I][int(SS)];
              // forward: y+ += A x+ - B x-, y- += B x+ + A x-
              // adjoint: y+ += A^T g+ + B^T g-, y- += -B^T g+ + A^T g-
              yp[I] = mfma(am, ADJ ? b_w : -b_w, yp[I]);
              ym[I] = mfma(ap, ADJ ? -b_w : b_w, ym[I]);
              ym[I] = mfma(am, a_w, ym[I]);
            }
          });
        });
      };
      v4f wa0[NA], wb0[NB], wa1[NA], wb1[NB];
      load_w(0, wa0, wb0);
#pragma unroll 1
      for (int g = 0; g < NG; g += 2) {
        if (g + 1 < NG) load_w(g + 1, wa1, wb1);
        run_group(g, wa0, wb0);
        if (g + 1 >= NG) break;
        if (g + 2 < NG) load_w(g + 2, wa0, wb0);
        run_group(g + 1, wa1, wb1);
      }
    }
    __syncthreads();
    if constexpr (NTW > 0) {
      so2_for<NTW>([&](auto I) {
        const int n = (WV + 2 * int(I)) * 16 + er;
        const int l3 = m + n / C, c3 = n % C;
        float* t3 = &tile[C * l3 * l3 + c3 * (2 * l3 + 1) + l3];
        so2_for<4>([&](auto R) {
          const int e = 4 * kq + int(R);
          t3[e * S::PAD + m] = yp[I][int(R)];
          if constexpr (m > 0) t3[e * S::PAD - m] = ym[I][int(R)];
        });
      });
    }
  });
}

// One CSR row per block of two wavefronts sharing the chunk's LDS tile (two
// rows' blocks fit a SIMD pair's LDS, so each SIMD holds two wavefronts).
// Wavefront w rotates and inverse-rotates edges 8w .. 8w + 7 of each chunk
// and runs half of the n-tiles; the two row sums meet in LDS at the end.
//
// FRAMES: the same rotation and maps, then, instead of the inverse rotation,
// the gradient with respect to the chunk's Wigner blocks.  With V the row's
// own vector (grad_out of the destination row over the destination-sorted
// rows, x of the source row over the source-sorted rows with the adjoint
// maps), the tile holds y~ (resp. dx~) and
//   gD[e]^l[m][n] (+)= sum_c tile[e][l][c][m] V[l][c][n],
// which is grad_D's y~ G^T (resp. dx~ x^T) term: out is then gD [E][ND],
// indexed by edge id, overwritten or (accumulate) added to.
//
// TWO: the inverse rotation uses other blocks, Dr, than the rotation on
// gather (D_e^T replaced by Dr_e^T): the terms of the mixed second
// derivatives through the frames, where one of the two places holds the
// frames' derivative.
template <int L, int C, bool ADJ, bool FRAMES, bool TWO = false>
__global__ __launch_bounds__(128, 2) void k_so2_conv(const int32_t* __restrict__ row_ptr,
                                                     const int32_t* __restrict__ col, const int32_t* __restrict__ eid,
                                                     const int32_t* __restrict__ order, const float* __restrict__ X,
                                                     const float* __restrict__ Dm, const float* __restrict__ W,
                                                     float* __restrict__ out, const int accumulate,
                                                     const float* __restrict__ V, const float* __restrict__ Dr) {
  using S = So2Shape<L, C>;
  static_assert(S::NACC * 64 <= S::kEdges * S::PAD, "row-sum exchange must fit the tile");
  static_assert(!(TWO && FRAMES), "two rotations only in the plain convolution");
  __shared__ float tile[S::kEdges * S::PAD];
  __shared__ float dl[S::kEdges * S::NDP];
  __shared__ float vrow[FRAMES ? S::DN : 1];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int c = lane % C, h = lane / C;
  const int row = order[blockIdx.x];
  const int beg = row_ptr[row], end = row_ptr[row + 1];
  float acc[S::NACC];
  so2_for<S::NACC>([&](auto I) { acc[I] = 0.f; });
  if constexpr (FRAMES) {
    for (int q = threadIdx.x; q < S::DN; q += 128) vrow[q] = V[(int64_t)row * S::DN + q];
  }

  for (int k0 = beg; k0 < end; k0 += S::kEdges) {
    const int ne = min(S::kEdges, end - k0);
    const int my_n = lane < ne ? col[k0 + lane] : 0;
    // the chunk's Wigner rows (zeros past the row end, so those edges rotate to zero)
    const int my_id = lane < ne ? eid[k0 + lane] : 0;
    load_wigner<L, C, 128>(threadIdx.x, ne, my_id, Dm, dl);
    __syncthreads();
    for (int e0 = 8 * wave; e0 < 8 * wave + 8; e0 += 4) {  // wave-uniform; four edges' loads issued together
      float xv[4][S::NC];
      so2_for<4>([&](auto I) {
        load_channel<L, C>(X + (int64_t)__builtin_amdgcn_readlane(my_n, e0 + int(I)) * S::DN, c, xv[I]);
      });
      so2_for<4>([&](auto I) {
        const int e = e0 + int(I);
        rotate_in<L, C>(xv[I], &dl[e * S::NDP], &tile[e * S::PAD], c, h);
      });
    }
    __syncthreads();
    // TWO: the inverse rotation's blocks replace the gather's in LDS (no
    // wavefront reads them again this chunk), loaded while the maps run
    if constexpr (TWO) load_wigner<L, C, 128>(threadIdx.x, ne, my_id, Dr, dl);
    if (wave == 0)
      so2_maps<L, C, ADJ, 0>(tile, W, lane);
    else
      so2_maps<L, C, ADJ, 1>(tile, W, lane);
    __syncthreads();

    if constexpr (FRAMES) {
      // entry r = (l, m, n) of edge e: thread q covers q, q + 128, ...
      for (int q = threadIdx.x; q < ne * S::ND; q += 128) {
        const int e = q / S::ND;
        int r = q - e * S::ND, l = 0;
        while (r >= (2 * l + 1) * (2 * l + 1)) {
          r -= (2 * l + 1) * (2 * l + 1);
          ++l;
        }
        const int n2 = 2 * l + 1, m = r / n2, n = r - m * n2;
        const float* te = &tile[e * S::PAD + C * l * l + m];
        const float* ve = &vrow[C * l * l + n];
        float sum = 0.f;
#pragma unroll 8
        for (int cc = 0; cc < C; ++cc) sum = fmaf(te[cc * n2], ve[cc * n2], sum);
        float* o = &out[(int64_t)eid[k0 + e] * S::ND + (q - e * S::ND)];
        *o = accumulate ? *o + sum : sum;  // each edge has one row in each view
      }
      __syncthreads();
      continue;
    }

    // inverse rotation on reduction: lane (c, h) sums components n = h, h + NSPLIT, ...
    const int e_end = min(ne, 8 * wave + 8);
    for (int e = 8 * wave; e < e_end; ++e) {  // wave-uniform
      const float* te = &tile[e * S::PAD];
      const float* dle = &dl[e * S::NDP];  // TWO: the blocks of Dr by now
      so2_for<L + 1>([&](auto IL) {
        constexpr int l = IL, n2 = 2 * l + 1;
        float yv[n2];
        so2_for<n2>([&](auto M) { yv[M] = te[S::xoff(l) + c * n2 + M]; });
        so2_for<S::J(l)>([&](auto JJ) {
          const int n = h + S::NSPLIT * int(JJ);
          if (n < n2) {
            float sum = acc[S::jbase(l) + JJ];
            so2_for<n2>([&](auto M) { sum = fmaf(dle[S::doff(l) + M * n2 + n], yv[M], sum); });
            acc[S::jbase(l) + JJ] = sum;
          }
        });
      });
    }
    __syncthreads();
  }

  if constexpr (FRAMES) return;
  // the two wavefronts' row sums (wavefront 1's through the tile), written once
  if (wave == 1) so2_for<S::NACC>([&](auto I) { tile[int(I) * 64 + lane] = acc[I]; });
  __syncthreads();
  if (wave == 0) {
    so2_for<S::NACC>([&](auto I) { acc[I] += tile[int(I) * 64 + lane]; });
    float* orow = out + (int64_t)row * S::DN;
    so2_for<L + 1>([&](auto IL) {
      constexpr int l = IL, n2 = 2 * l + 1;
      so2_for<S::J(l)>([&](auto JJ) {
        const int n = h + S::NSPLIT * int(JJ);
        if (n < n2) {
          float* o = &orow[S::xoff(l) + c * n2 + n];
          *o = accumulate ? *o + acc[S::jbase(l) + JJ] : acc[S::jbase(l) + JJ];  // the row's only writer
        }
      });
    });
  }
}

__global__ __launch_bounds__(256) void k_so2_fill_zero(int64_t n, float* __restrict__ p) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

// out = a + b (the two terms of the map gradient of the mixed second
// derivatives through the frames)
__global__ __launch_bounds__(256) void k_so2_add(int64_t n, const float* __restrict__ a, const float* __restrict__ b,
                                                 float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = a[i] + b[i];
}

// dDp_e = dD_e - c_e J D_e, with J the generator of rolls about the edge
// axis on each degree-l block ((J v)[l - m] = m v[l + m] and
// (J v)[l + m] = -m v[l - m] for m > 0) and c_e = <dD_e, J D_e> / |J D_e|^2,
// computed in fp64 and rounded once.  A roll of an edge's frame about its
// axis leaves the convolution unchanged, so the derivatives through the
// frames are blind to any dD along J D_e: the mixed second derivatives with
// dDp equal those with dD exactly (for any c_e), and dDp no longer carries
// the roll rate of a frames' derivative, which grows without bound near the
// frame construction's pole and whose two terms cancel.  Edges in blocks of
// 64, staged through LDS so that the global accesses are coalesced; the first
// wavefront projects one edge per lane.
template <int L>
__global__ __launch_bounds__(256) void k_so2_unroll(int64_t n_edges, const float* __restrict__ D,
                                                    const float* __restrict__ dD, float* __restrict__ out) {
  constexpr int ND = (L + 1) * (2 * L + 1) * (2 * L + 3) / 3;
  constexpr int EB = 64;
  __shared__ float sD[EB * ND];
  __shared__ float sd[EB * ND];
  const int64_t e0 = (int64_t)blockIdx.x * EB;
  const int ne = (int)min((int64_t)EB, n_edges - e0);
  const int64_t base = e0 * ND;
  const int cnt = ne * ND;
  for (int i = threadIdx.x; i < cnt; i += 256) {
    sD[i] = D[base + i];
    sd[i] = dD[base + i];
  }
  __syncthreads();
  if ((int)threadIdx.x < ne) {
    const float* a = sD + threadIdx.x * ND;
    float* b = sd + threadIdx.x * ND;
    double num = 0.0, den = 0.0;
    so2_for<L>([&](auto lm1) {
      constexpr int l = decltype(lm1)::value + 1;
      constexpr int off = l * (2 * l - 1) * (2 * l + 1) / 3;
      constexpr int w = 2 * l + 1;
      for (int m = 1; m <= l; ++m)
        for (int n = 0; n < w; ++n) {
          const double ap = a[off + (l + m) * w + n], am = a[off + (l - m) * w + n];
          num += m * ((double)b[off + (l - m) * w + n] * ap - (double)b[off + (l + m) * w + n] * am);
          den += (double)(m * m) * (ap * ap + am * am);
        }
    });
    const double c = den > 0.0 ? num / den : 0.0;
    so2_for<L>([&](auto lm1) {
      constexpr int l = decltype(lm1)::value + 1;
      constexpr int off = l * (2 * l - 1) * (2 * l + 1) / 3;
      constexpr int w = 2 * l + 1;
      for (int m = 1; m <= l; ++m)
        for (int n = 0; n < w; ++n) {
          const double ap = a[off + (l + m) * w + n], am = a[off + (l - m) * w + n];
          const double bp = b[off + (l + m) * w + n], bm = b[off + (l - m) * w + n];
          b[off + (l + m) * w + n] = (float)(bp + c * m * am);
          b[off + (l - m) * w + n] = (float)(bm - c * m * ap);
        }
    });
  }
  __syncthreads();
  for (int i = threadIdx.x; i < cnt; i += 256) out[base + i] = sd[i];
}

// Each map block of W transposed in place of itself: Wt[off + n K + k] =
// W[off + k K + n] (the adjoint kernel's weights).
template <int L, int C>
__global__ __launch_bounds__(256) void k_so2_transpose(const float* __restrict__ W, float* __restrict__ Wt) {
  using S = So2Shape<L, C>;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= S::NW) return;
  int off = 0, K = 0;
  for (int m = 0; m <= L; ++m) {
    const int k = S::K(m), n = (m ? 2 : 1) * k * k;
    if (idx < off + n) {
      K = k;
      if (idx >= off + k * k) off += k * k;  // B_m
      break;
    }
    off += n;
  }
  const int r = idx - off, n = r / K, k = r - n * K;
  Wt[idx] = W[off + k * K + n];
}

// row of CSR slot k: the last r with row_ptr[r] <= k
__device__ __forceinline__ int slot_row(const int32_t* __restrict__ row_ptr, int n_rows, int k) {
  int lo = 0, hi = n_rows - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (row_ptr[mid] <= k)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

template <int L, int C, int WV, bool TWO>
__device__ __forceinline__ void wgrad_wave(int n_rows, int64_t s0, int64_t s1, const int32_t* __restrict__ row_ptr,
                                           const int32_t* __restrict__ col, const int32_t* __restrict__ eid,
                                           const float* __restrict__ X, const float* __restrict__ G,
                                           const float* __restrict__ Dm, const float* __restrict__ Dg,
                                           float* __restrict__ part, float* xt, float* gt, float* dl, float* dl2) {
  using S = So2Shape<L, C>;
  constexpr int NMINE = So2Jobs<L, C>::value.nmine[WV];
  const int lane = threadIdx.x & 63;
  const int c = lane % C, h = lane / C;
  const int er = lane & 15, kq = lane >> 4;
  v4f accA[NMINE > 0 ? NMINE : 1], accB[NMINE > 0 ? NMINE : 1];  // a wavefront may own no tile
  so2_for<NMINE>([&](auto I) {
    accA[I] = v4f{0.f, 0.f, 0.f, 0.f};
    accB[I] = v4f{0.f, 0.f, 0.f, 0.f};
  });

  // destination row of the block's current slot: one search, then a cursor
  int cur = s0 < s1 ? slot_row(row_ptr, n_rows, (int)s0) : 0;
  for (int64_t k0 = s0; k0 < s1; k0 += S::kEdges) {
    const int ne = (int)min<int64_t>(S::kEdges, s1 - k0);
    int my_s = 0, my_d = 0, my_id = 0;
    if (er < ne) {
      const int k = (int)(k0 + er);
      my_s = col[k];
      my_id = eid[k];
      int r = cur;
      while (row_ptr[r + 1] <= k) ++r;  // ends: row_ptr[n_rows] = n_slots > k
      my_d = r;
    }
    cur = __builtin_amdgcn_readlane(my_d, ne - 1);
    load_wigner<L, C, 64 * S::kWaves>(threadIdx.x, ne, my_id, Dm, dl);
    if constexpr (TWO) load_wigner<L, C, 64 * S::kWaves>(threadIdx.x, ne, my_id, Dg, dl2);
    __syncthreads();
    {  // this wavefront's two edges, x and grad_out rows loaded together
      float xv[2][S::NC], gv[2][S::NC];
      so2_for<2>([&](auto I) {
        constexpr int e = WV + S::kWaves * int(I);
        load_channel<L, C>(X + (int64_t)__builtin_amdgcn_readlane(my_s, e) * S::DN, c, xv[I]);
        load_channel<L, C>(G + (int64_t)__builtin_amdgcn_readlane(my_d, e) * S::DN, c, gv[I]);
      });
      so2_for<2>([&](auto I) {
        constexpr int e = WV + S::kWaves * int(I);
        rotate_in<L, C>(xv[I], &dl[e * S::NDP], &xt[e * S::PADW], c, h);
        rotate_in<L, C>(gv[I], TWO ? &dl2[e * S::NDP] : &dl[e * S::NDP], &gt[e * S::PADW], c, h);
      });
    }
    __syncthreads();
    so2_for<NMINE>([&](auto I) {
      constexpr typename S::Job jb = S::job(So2Jobs<L, C>::value.list[WV][int(I)]);
      constexpr int m = jb.m;
      const int o = jb.ot * 16 + er, i = jb.it * 16 + er;
      const int lo = m + o / C, co = o % C, li = m + i / C, ci = i % C;
      const float* go = &gt[C * lo * lo + co * (2 * lo + 1) + lo];
      const float* xi = &xt[C * li * li + ci * (2 * li + 1) + li];
      so2_for<4>([&](auto KS) {
        const int e = 4 * int(KS) + kq;  // K index of both fragments: the edge
        const float gp = go[e * S::PADW + m], xp = xi[e * S::PADW + m];
        accA[I] = mfma(gp, xp, accA[I]);
        if constexpr (m > 0) {
          const float gm = go[e * S::PADW - m], xm = xi[e * S::PADW - m];
          accA[I] = mfma(gm, xm, accA[I]);   // dA += g+ x+^T + g- x-^T
          accB[I] = mfma(gm, xp, accB[I]);   // dB += g- x+^T - g+ x-^T
          accB[I] = mfma(-gp, xm, accB[I]);
        }
      });
    });
    __syncthreads();
  }

  float* pb = part + (int64_t)blockIdx.x * S::NW;
  so2_for<NMINE>([&](auto I) {
    constexpr typename S::Job jb = S::job(So2Jobs<L, C>::value.list[WV][int(I)]);
    constexpr int m = jb.m, K = S::K(m);
    const int i = jb.it * 16 + er;
    so2_for<4>([&](auto R) {
      const int o = jb.ot * 16 + 4 * kq + int(R);
      pb[S::woffA(m) + o * K + i] = accA[I][int(R)];
      if constexpr (m > 0) pb[S::woffB(m) + o * K + i] = accB[I][int(R)];
    });
  });
}

// TWO: grad_out rotated by other blocks, Dg, than x (the mixed second
// derivatives through the frames).
template <int L, int C, bool TWO = false>
__global__ __launch_bounds__(512) void k_so2_wgrad(int n_rows, int64_t n_slots, int64_t per_block,
                                                   const int32_t* __restrict__ row_ptr,
                                                   const int32_t* __restrict__ col, const int32_t* __restrict__ eid,
                                                   const float* __restrict__ X, const float* __restrict__ G,
                                                   const float* __restrict__ Dm, const float* __restrict__ Dg,
                                                   float* __restrict__ part) {
  using S = So2Shape<L, C>;
  __shared__ float xt[S::kEdges * S::PADW];
  __shared__ float gt[S::kEdges * S::PADW];
  __shared__ float dl[S::kEdges * S::NDP];
  __shared__ float dl2[TWO ? S::kEdges * S::NDP : 1];
  const int64_t s0 = (int64_t)blockIdx.x * per_block;
  const int64_t s1 = min(n_slots, s0 + per_block);
  switch (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) {
    case 0: wgrad_wave<L, C, 0, TWO>(n_rows, s0, s1, row_ptr, col, eid, X, G, Dm, Dg, part, xt, gt, dl, dl2); break;
    case 1: wgrad_wave<L, C, 1, TWO>(n_rows, s0, s1, row_ptr, col, eid, X, G, Dm, Dg, part, xt, gt, dl, dl2); break;
    case 2: wgrad_wave<L, C, 2, TWO>(n_rows, s0, s1, row_ptr, col, eid, X, G, Dm, Dg, part, xt, gt, dl, dl2); break;
    case 3: wgrad_wave<L, C, 3, TWO>(n_rows, s0, s1, row_ptr, col, eid, X, G, Dm, Dg, part, xt, gt, dl, dl2); break;
    case 4: wgrad_wave<L, C, 4, TWO>(n_rows, s0, s1, row_ptr, col, eid, X, G, Dm, Dg, part, xt, gt, dl, dl2); break;
    case 5: wgrad_wave<L, C, 5, TWO>(n_rows, s0, s1, row_ptr, col, eid, X, G, Dm, Dg, part, xt, gt, dl, dl2); break;
    case 6: wgrad_wave<L, C, 6, TWO>(n_rows, s0, s1, row_ptr, col, eid, X, G, Dm, Dg, part, xt, gt, dl, dl2); break;
    default: wgrad_wave<L, C, 7, TWO>(n_rows, s0, s1, row_ptr, col, eid, X, G, Dm, Dg, part, xt, gt, dl, dl2); break;
  }
}

// grad_w[j] = sum over blocks b (in order) of part[b][j]
__global__ __launch_bounds__(256) void k_so2_wsum(int nb, int64_t nw, const float* __restrict__ part,
                                                  float* __restrict__ gw) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= nw) return;
  double s = 0.0;
#pragma unroll 8
  for (int b = 0; b < nb; ++b) s += part[(int64_t)b * nw + j];
  gw[j] = (float)s;
}

template <int L, int C>
hipError_t conv_LC(bool adjoint, bool accumulate, int n_rows, const int32_t* row_ptr, const int32_t* col,
                   const int32_t* eid, const int32_t* order, const float* X, const float* D, const float* W,
                   float* out, float* Wt, const float* V, const float* Dr, hipStream_t s) {
  using S = So2Shape<L, C>;
  const dim3 grid((unsigned)n_rows), block(128);
  const int acc = (int)accumulate;
  if (adjoint) {
    hipLaunchKernelGGL((k_so2_transpose<L, C>), dim3((unsigned)((S::NW + 255) / 256)), dim3(256), 0, s, W, Wt);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (V != nullptr)
      hipLaunchKernelGGL((k_so2_conv<L, C, true, true>), grid, block, 0, s, row_ptr, col, eid, order, X, D, Wt, out,
                         acc, V, Dr);
    else if (Dr != nullptr)
      hipLaunchKernelGGL((k_so2_conv<L, C, true, false, true>), grid, block, 0, s, row_ptr, col, eid, order, X, D,
                         Wt, out, acc, V, Dr);
    else
      hipLaunchKernelGGL((k_so2_conv<L, C, true, false>), grid, block, 0, s, row_ptr, col, eid, order, X, D, Wt, out,
                         acc, V, Dr);
  } else {
    if (V != nullptr)
      hipLaunchKernelGGL((k_so2_conv<L, C, false, true>), grid, block, 0, s, row_ptr, col, eid, order, X, D, W, out,
                         acc, V, Dr);
    else if (Dr != nullptr)
      hipLaunchKernelGGL((k_so2_conv<L, C, false, false, true>), grid, block, 0, s, row_ptr, col, eid, order, X, D,
                         W, out, acc, V, Dr);
    else
      hipLaunchKernelGGL((k_so2_conv<L, C, false, false>), grid, block, 0, s, row_ptr, col, eid, order, X, D, W, out,
                         acc, V, Dr);
  }
  return hipGetLastError();
}

template <int L, int C>
hipError_t wgrad_LC(int n_rows, int64_t n_slots, int nb, const int32_t* row_ptr, const int32_t* col,
                    const int32_t* eid, const float* X, const float* G, const float* D, const float* Dg, float* part,
                    float* gw, hipStream_t s) {
  using S = So2Shape<L, C>;
  const int64_t per_block = (n_slots + nb - 1) / nb;
  if (Dg != nullptr)
    hipLaunchKernelGGL((k_so2_wgrad<L, C, true>), dim3((unsigned)nb), dim3(64 * S::kWaves), 0, s, n_rows, n_slots,
                       per_block, row_ptr, col, eid, X, G, D, Dg, part);
  else
    hipLaunchKernelGGL((k_so2_wgrad<L, C>), dim3((unsigned)nb), dim3(64 * S::kWaves), 0, s, n_rows, n_slots,
                       per_block, row_ptr, col, eid, X, G, D, D, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_so2_wsum, dim3((unsigned)((S::NW + 255) / 256)), dim3(256), 0, s, nb, (int64_t)S::NW, part,
                     gw);
  return hipGetLastError();
}

}  // namespace

int64_t so2_weight_numel(int L, int C) {
  int64_t n = 0;
  for (int m = 0; m <= L; ++m) n += (m ? 2 : 1) * int64_t((L + 1 - m) * C) * ((L + 1 - m) * C);
  return n;
}

int so2_wgrad_blocks(int64_t n_edges) {
  const int64_t nb = (n_edges + 63) / 64;
  return (int)(nb < 1 ? 1 : (nb > 512 ? 512 : nb));
}

#define SO2_CASES(F, ...)                                   \
  switch (L * 100 + C) {                                    \
    case 116: return F<1, 16>(__VA_ARGS__);                 \
    case 132: return F<1, 32>(__VA_ARGS__);                 \
    case 216: return F<2, 16>(__VA_ARGS__);                 \
    case 232: return F<2, 32>(__VA_ARGS__);                 \
    case 316: return F<3, 16>(__VA_ARGS__);                 \
    case 332: return F<3, 32>(__VA_ARGS__);                 \
    default: return hipErrorInvalidValue;                   \
  }

hipError_t launch_so2_conv(int L, int C, bool adjoint, bool accumulate, int n_rows, const int32_t* row_ptr,
                           const int32_t* col, const int32_t* eid, const int32_t* order, const float* X,
                           const float* D, const float* W, float* out, float* Wt, const float* V, hipStream_t s,
                           const float* Dr) {
  if (n_rows <= 0) return hipSuccess;
  SO2_CASES(conv_LC, adjoint, accumulate, n_rows, row_ptr, col, eid, order, X, D, W, out, Wt, V, Dr, s)
}

hipError_t launch_so2_wgrad(int L, int C, int n_rows, int64_t n_edges, const int32_t* row_ptr, const int32_t* col,
                            const int32_t* eid, const float* X, const float* G, const float* D, float* part,
                            float* grad_w, int max_blocks, hipStream_t s, const float* Dg) {
  int nb = so2_wgrad_blocks(n_edges);
  if (max_blocks > 0 && nb > max_blocks) nb = max_blocks;
  SO2_CASES(wgrad_LC, n_rows, n_edges, nb, row_ptr, col, eid, X, G, D, Dg, part, grad_w, s)
}

// Device scratch of tpconv_so2_backward_noalloc (callers that cannot
// allocate): the transposed maps, then one partial map gradient per block of
// edges.  Each device that runs the library holds its own copy until the
// process ends; every call on a device shares it.
constexpr int64_t kSo2ScratchFloats = int64_t(1) << 22;  // 16 MiB
static __device__ __align__(256) float scratch[kSo2ScratchFloats];

// This device's address of the scratch array, looked up once per device (the
// array's name is a host-side stand-in, not a device address).
hipError_t so2_scratch(float** ptr, int64_t* n_floats) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static float* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = static_cast<float*>(p);
  }
  *ptr = addr[dev];
  *n_floats = kSo2ScratchFloats;
  return hipSuccess;
}

hipError_t launch_so2_add(int64_t n, const float* a, const float* b, float* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_so2_add, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, n, a, b, out);
  return hipGetLastError();
}

hipError_t launch_so2_unroll(int L, int64_t n_edges, const float* D, const float* dD, float* out, hipStream_t s) {
  if (n_edges <= 0) return hipSuccess;
  const dim3 grid((unsigned)((n_edges + 63) / 64)), block(256);
  switch (L) {
    case 1: hipLaunchKernelGGL(k_so2_unroll<1>, grid, block, 0, s, n_edges, D, dD, out); break;
    case 2: hipLaunchKernelGGL(k_so2_unroll<2>, grid, block, 0, s, n_edges, D, dD, out); break;
    case 3: hipLaunchKernelGGL(k_so2_unroll<3>, grid, block, 0, s, n_edges, D, dD, out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_so2_fill_zero(int64_t n, float* p, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_so2_fill_zero, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, n, p);
  return hipGetLastError();
}

}  // namespace tpconv
