// tp_common.hpp -- shared declarations between the host API and the kernels.
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime_api.h>

#include "cg_real.hpp"

namespace tpconv {

constexpr int kMaxL = cg::kLMax;

// Triples (l1, l2, l3) with all l <= L and the triangle rule, enumerated in
// lexicographic order; the kernels index per-path data by this id.
constexpr int triple_count(int L) {
  int n = 0;
  for (int a = 0; a <= L; ++a)
    for (int b = 0; b <= L; ++b)
      for (int c = 0; c <= L; ++c)
        if (cg::triangle(a, b, c)) ++n;
  return n;
}

constexpr int triple_id(int L, int l1, int l2, int l3) {
  int n = 0;
  for (int a = 0; a <= L; ++a)
    for (int b = 0; b <= L; ++b)
      for (int c = 0; c <= L; ++c)
        if (cg::triangle(a, b, c)) {
          if (a == l1 && b == l2 && c == l3) return n;
          ++n;
        }
  return -1;
}

constexpr int kMaxTriples = triple_count(kMaxL);  // 65
static_assert(kMaxTriples <= 128, "triple ids must fit the two path-mask words");

// Launch arguments shared by all kernels.  `row_ptr`, `col` and `eid` are the
// CSR view the kernel walks: destination-sorted for the forward and the
// double backward's grad_G (col = src), source-sorted for the backward and
// the double backward's grad_x / grad_Y / grad_W (col = dst).
struct KernelArgs {
  int32_t n_rows;       // nodes
  int32_t mul;          // U, channels per segment (1..64)
  int32_t lps_log2;     // log2 of lanes per edge slot: next power of two >= U
  int32_t nslots;       // edges a wave processes side by side: 64 >> lps_log2
  int32_t d_in, d_out, d_sh;
  int32_t from_vec;     // 1: the kernels evaluate Y from the edge vectors `vec` themselves (full plans)
  int64_t wstride;      // weight_numel
  uint64_t pmask_lo;    // bit t: triple t is a path of the plan (t < 64)
  uint64_t pmask_hi;    // bit t-64
  uint64_t first3_lo;   // bit t: path t is the first path (in (l1, l2, l3) order) into its output l
  uint64_t first3_hi;
  uint64_t first1_lo;   // bit t: path t is the first path (in (l3, l1, l2) order) out of its input l
  uint64_t first1_hi;
  int32_t out_l_mask;   // bit l: some path writes output l
  int32_t in_l_mask;    // bit l: some path reads input l
  int32_t full_plan;    // 1: segments l = 0..L in order with parity (-1)^l in and out, SH l <= L,
                        //    so the plan holds every even-sum triple in triple order
  int32_t acc;          // run-time plans: bit 0 adds into `out` instead of overwriting it, bit 1 into dY
                        //    (the later passes of a plan with both parities of one l)
  const int32_t* row_ptr;
  const int32_t* col;
  const int32_t* eid;
  const int32_t* order; // rows in the order wavefronts take them (longest first)
  int32_t in_off[kMaxL + 1];   // x column of segment with this l, -1 if absent
  int32_t out_off[kMaxL + 1];  // out column of segment with this l, -1 if absent
  int32_t woff[kMaxTriples];   // W column of path with this triple, -1 if absent
  const void* x;
  const void* Y;
  const void* W;
  const void* G;        // backward kernels only
  const void* xa;       // double backward: cotangent of grad_x, like x (null = zero)
  const void* Yb;       // double backward: cotangent of grad_Y, like Y (null = zero)
  const void* Wc;       // double backward: cotangent of grad_W, like W (null = zero)
  void* out;            // forward: out; backward: grad_x; double backward: grad_G or grad_x (may be null)
  void* dY;             // backward kernels: grad_Y (may be null)
  void* dW;             // backward kernels: grad_W (may be null)
  const void* vec;      // from_vec: the edge vectors [E][3] (Y unused)
  void* gvec;           // backward with vec: grad_vec [E][3] in place of grad_Y (may be null)
};

// Launchers, one per (lmax, dtype), defined by tp_kernels.hip compiled once
// per (lmax, dtype, TPCONV_DD): fwd/bwd with TPCONV_DD=0, and the double
// backward's two passes ddf (grad_G) / ddb (grad_x, grad_Y, grad_W) with 1;
// radial: the forward (fwd) or backward with W = h M generated in-kernel
// (fp32 units with TPCONV_DD=0, compile-time plans only).
#define TPCONV_DECLARE_LAUNCHERS(L)                                                \
  hipError_t launch_fwd_l##L##_f32(const KernelArgs& a, hipStream_t s);            \
  hipError_t launch_fwd_l##L##_f64(const KernelArgs& a, hipStream_t s);            \
  hipError_t launch_bwd_l##L##_f32(const KernelArgs& a, hipStream_t s);            \
  hipError_t launch_bwd_l##L##_f64(const KernelArgs& a, hipStream_t s);            \
  hipError_t launch_ddf_l##L##_f32(const KernelArgs& a, hipStream_t s);            \
  hipError_t launch_ddf_l##L##_f64(const KernelArgs& a, hipStream_t s);            \
  hipError_t launch_ddb_l##L##_f32(const KernelArgs& a, hipStream_t s);            \
  hipError_t launch_ddb_l##L##_f64(const KernelArgs& a, hipStream_t s);            \
  hipError_t launch_radial_l##L##_f32(bool fwd, const KernelArgs& a, const float* h, const float* M,  \
                                      float* dh, int lgH, hipStream_t s);

TPCONV_DECLARE_LAUNCHERS(0)
TPCONV_DECLARE_LAUNCHERS(1)
TPCONV_DECLARE_LAUNCHERS(2)
TPCONV_DECLARE_LAUNCHERS(3)
TPCONV_DECLARE_LAUNCHERS(4)

// Edge harmonics, their gradient and the position gradient (sh.hip).
// SO(2) convolution (so2.hip, sh.hip)
hipError_t launch_so2_wigner(int L, bool f64, int64_t n_edges, const void* vec, void* D, hipStream_t s);
int64_t so2_weight_numel(int L, int C);
int so2_wgrad_blocks(int64_t n_edges);
// accumulate: out += instead of out = (each row has one writer, so still deterministic).
// Wt: adjoint only, weight_numel floats.  V non-null: the frame-gradient mode, out = grad_D
// [E][sum (2l+1)^2] by edge id, V the rows' own vectors (grad_out, or x for the adjoint).
// Dr non-null (V null): the inverse rotation uses Dr instead of D.
hipError_t launch_so2_conv(int L, int C, bool adjoint, bool accumulate, int n_rows, const int32_t* row_ptr,
                           const int32_t* col, const int32_t* eid, const int32_t* order, const float* X,
                           const float* D, const float* W, float* out, float* Wt, const float* V, hipStream_t s,
                           const float* Dr = nullptr);
hipError_t launch_so2_wigner_backward(int L, bool f64, int64_t n_edges, const void* vec, const void* grad_D,
                                      void* grad_vec, hipStream_t s);
// the frames' directional derivative along dvec [E][3]: dD [E][sum (2l+1)^2]
hipError_t launch_so2_wigner_jvp(int L, bool f64, int64_t n_edges, const void* vec, const void* dvec, void* dD,
                                 hipStream_t s);
// out = a + b
hipError_t launch_so2_add(int64_t n, const float* a, const float* b, float* out, hipStream_t s);
// dDp = dD minus, per edge, its component along the frame's roll about the
// edge axis (fp64 projection), lmax 1..3.
hipError_t launch_so2_unroll(int L, int64_t n_edges, const float* D, const float* dD, float* out, hipStream_t s);
hipError_t launch_so2_fill_zero(int64_t n, float* p, hipStream_t s);
// max_blocks > 0 caps the number of edge blocks (and of partial sums in part); Dg non-null:
// grad_out rotated by Dg instead of D
hipError_t launch_so2_wgrad(int L, int C, int n_rows, int64_t n_edges, const int32_t* row_ptr, const int32_t* col,
                            const int32_t* eid, const float* X, const float* G, const float* D, float* part,
                            float* grad_w, int max_blocks, hipStream_t s, const float* Dg = nullptr);
// the allocation-free backward's device scratch on the current device
hipError_t so2_scratch(float** ptr, int64_t* n_floats);
hipError_t launch_sh(int L, bool f64, int64_t n_edges, const void* vec, void* Y, hipStream_t s);
hipError_t launch_sh_backward(int L, bool f64, int64_t n_edges, const void* vec, const void* grad_Y, void* grad_vec,
                              hipStream_t s);
hipError_t launch_pos_backward(bool f64, int64_t n_nodes, const int32_t* src_row, const int32_t* src_eid,
                               const int32_t* dst_row, const int32_t* dst_eid, const void* grad_vec, void* grad_pos,
                               hipStream_t s);

}  // namespace tpconv
