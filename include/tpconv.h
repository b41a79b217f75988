/*
 * tpconv.h -- C ABI of the MI355X (gfx950) Clebsch-Gordan tensor-product
 * convolution library, libtpconv.so.
 *
 * The operation is the "CGTP convolution" of equivariant interatomic
 * potentials (LunaTP: Enabling Efficient and Scalable Tensor Product for
 * Equivariant MLIPs -- Abstract): a tensor-product layer and its following
 * reduce layer over a sparse Clebsch-Gordan coefficient matrix (FlashTP:
 * Fused, Sparsity-Aware Tensor Product for Machine Learning Interatomic
 * Potentials -- "Problem" and "Approach").  For an edge e with j = src(e),
 * i = dst(e), a path p = (s1, l2, s3) of real-basis CG tensor C_p and a
 * channel u:
 *
 *   out[i,s3,u,m3] = sum_{e: dst=i} sum_{p->s3} W[e,p,u]
 *                    sum_{m1,m2} C_p[m1,m2,m3] x[j,s1,u,m1] Y[e,l2,m2]
 *
 * and the backward gives dx, dY, dW of <G, out> for a supplied G.  Where
 * the pages are silent the library takes these readings: channelwise (uvu)
 * coupling, one weight per (edge, path, channel), paths into the same
 * output segment summed with coefficient 1, complex CG from Racah's formula
 * (Condon-Shortley phase) turned real through the basis change U^l listed
 * in cg_real.hpp, odd l1+l2+l3 taking the imaginary part.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensor pointers are DEVICE pointers in the plan's dtype, row-major and
 *    contiguous:
 *      x   [N][D_in]    segments concatenated in irreps order; segment s
 *                       stored [mul_s][2 l_s + 1], m ascending -l..l
 *      Y   [E][D_sh]    D_sh = (sh_lmax+1)^2, (l, m) at column l*l + l + m
 *      W   [E][weight_numel]  path p at columns [off_p, off_p + mul_p),
 *                       paths in lexicographic (s1, l2, s3) order
 *      out [N][D_out]   like x
 *    Per-edge tensors are in the caller's edge order (the order of the
 *    src/dst arrays given to tpconv_graph_create).
 *  - Ownership: the caller owns every device buffer, including the graph
 *    workspace.  The library never allocates device memory.  Plans and
 *    graph handles own only small host structs.
 *  - Every call is asynchronous on `stream`, except tpconv_graph_create,
 *    which synchronises `stream` once to report index errors.
 *  - A status other than TPCONV_OK means nothing was launched; the message
 *    is available from tpconv_last_error() on the calling thread.  No C++
 *    exception crosses this interface.
 *  - Results are deterministic: the reductions use no floating-point
 *    atomics, so repeated calls give bitwise identical outputs.
 *
 * Kernel coverage: every irreps string may hold each (l, parity) at most
 * once (an l may appear with both parities, e.g. 32x1o+32x1e), all segments
 * of irreps_in and irreps_out share one multiplicity U with 1 <= U <= 64 (one
 * 64-lane wavefront holds a channel per lane), and every l (inputs, outputs,
 * SH) is at most TPCONV_MAX_L.  Other plans are rejected with
 * TPCONV_E_UNSUPPORTED.  A plan holding both parities of some l runs as up to
 * four launches per kernel (segments grouped by the type p (-1)^l on each
 * side), the later ones adding into the outputs the earlier ones wrote.
 */
#ifndef TPCONV_H
#define TPCONV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TPCONV_MAX_L 4

typedef enum { TPCONV_F32 = 0, TPCONV_F64 = 1 } tpconv_dtype;

typedef enum {
  TPCONV_OK = 0,
  TPCONV_E_INVALID_ARG = 1, /* NULL pointer, negative size, bad dtype, size mismatch */
  TPCONV_E_IRREPS = 2,      /* irreps string does not parse */
  TPCONV_E_UNSUPPORTED = 3, /* l > TPCONV_MAX_L, repeated (l, parity), unequal multiplicities, U > 64 */
  TPCONV_E_NO_PATHS = 4,    /* no admissible (s1, l2, s3) path */
  TPCONV_E_WORKSPACE = 5,   /* workspace (or the library's scratch) too small, or misaligned */
  TPCONV_E_INDEX = 6,       /* some src/dst index outside [0, n_nodes) */
  TPCONV_E_HIP = 7          /* a HIP runtime call or kernel launch failed */
} tpconv_status;

typedef struct tpconv_plan_s* tpconv_plan_t;
typedef struct tpconv_graph_s* tpconv_graph_t;

typedef struct {
  int64_t dim_in;        /* D_in  = sum mul*(2l+1) over irreps_in  */
  int64_t dim_out;       /* D_out = sum mul*(2l+1) over irreps_out */
  int64_t dim_sh;        /* (sh_lmax+1)^2 */
  int64_t n_paths;       /* P */
  int64_t weight_numel;  /* sum_p mul_p = row width of W and dW */
  int64_t cg_nnz;        /* nonzero real CG entries summed over the paths */
  int64_t cg_nvalues;    /* distinct |CG| values after deduplication */
  int64_t mul;           /* the common multiplicity U */
  int64_t kernel_lmax;   /* l bound the dispatched kernels are built for */
  int32_t dtype;         /* tpconv_dtype */
  int32_t reserved;
} tpconv_plan_info;

/* ---------------------------------------------------------------- plans --
 * tpconv_plan: parse the irreps, enumerate the admissible paths and build
 * the sparse real CG table (COO with deduplicated values), all on the host.
 * The sparse COO table with deduplicated values and the grouping of paths
 * that share an input follow FlashTP's "Approach" section and the path
 * aggregation rows of its measured-effects table.
 *   irreps_in, irreps_out: "mul x l p" terms joined by '+', e.g.
 *     "32x0e+32x1o+32x2e"; mul defaults to 1; p is 'e' or 'o'.
 *   sh_lmax: the SH input holds one copy of every l = 0..sh_lmax, parity (-1)^l.
 *   Path rule: |l1-l2| <= l3 <= l1+l2, p1 (-1)^l2 == p3, mul_s1 == mul_s3.
 * Errors: TPCONV_E_INVALID_ARG (NULL, sh_lmax < 0, bad dtype),
 *   TPCONV_E_IRREPS, TPCONV_E_UNSUPPORTED, TPCONV_E_NO_PATHS.
 * On success *out owns a host struct; free it with tpconv_plan_destroy. */
tpconv_status tpconv_plan(const char* irreps_in, int sh_lmax, const char* irreps_out,
                          tpconv_dtype dtype, tpconv_plan_t* out);

/* Sizes of a plan.  Errors: TPCONV_E_INVALID_ARG on NULL. */
tpconv_status tpconv_plan_query(tpconv_plan_t plan, tpconv_plan_info* info);

/* Path list, host buffer of n_paths*4 int32: (s1, l2, s3, weight column
 * offset) per path, in W's column order.  Errors: TPCONV_E_INVALID_ARG. */
tpconv_status tpconv_plan_paths(tpconv_plan_t plan, int32_t* paths);

/* The plan's sparse real CG table, host buffers:
 *   entries[cg_nnz]: packed u32  m1 | m2<<4 | m3<<8 | neg<<12 | value_index<<13
 *                    (m indices are m + l, 0..2l; value = (neg ? -1 : 1) *
 *                    values[value_index]); entries of a path are ordered by
 *                    (m1, m2, m3)
 *   path_ptr[n_paths+1]: entries of path p are [path_ptr[p], path_ptr[p+1])
 *   values[cg_nvalues]: distinct |C| in fp64.
 * Any pointer may be NULL to skip that array.  The kernels are compiled
 * from the same builder (cg_real.hpp), so these are the coefficients they
 * apply.  Errors: TPCONV_E_INVALID_ARG on a NULL plan. */
tpconv_status tpconv_plan_table(tpconv_plan_t plan, uint32_t* entries, int32_t* path_ptr,
                                double* values);

void tpconv_plan_destroy(tpconv_plan_t plan);

/* ---------------------------------------------------------------- graphs --
 * Destination-sorted and source-sorted CSR views of an edge list (node-
 * centric execution, LunaTP Abstract).  Rows are stable: inside a row,
 * edges keep the caller's order, so the layout and every result built on
 * it are deterministic.
 *
 * tpconv_graph_workspace_bytes: device bytes the caller must provide for
 * n_nodes nodes and n_edges edges (returns 0 for negative sizes). */
size_t tpconv_graph_workspace_bytes(int64_t n_nodes, int64_t n_edges);

/* tpconv_graph_create: build both CSR views on `stream` into `workspace`
 * (device, >= tpconv_graph_workspace_bytes, 256-byte aligned).
 *   src, dst: device int32 [n_edges]; edge e goes src[e] -> dst[e].
 * The workspace must outlive the graph and must not be written by the
 * caller while the graph is in use.  Edges with an index outside
 * [0, n_nodes) are dropped from the layout and reported: the call then
 * returns TPCONV_E_INDEX (after synchronising `stream`) and *out is NULL.
 * Other errors: TPCONV_E_INVALID_ARG (NULL, n_nodes < 0, n_edges < 0,
 * n_edges >= 2^31), TPCONV_E_WORKSPACE, TPCONV_E_HIP. */
tpconv_status tpconv_graph_create(int64_t n_nodes, int64_t n_edges, const int32_t* src,
                                  const int32_t* dst, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream, tpconv_graph_t* out);

/* Copy the CSR arrays to host buffers (any may be NULL), for inspection:
 * dst_row_ptr/src_row_ptr [n_nodes+1], dst_col (=src), dst_eid, src_col
 * (=dst), src_eid [n_edges].  Synchronous on `stream`. */
tpconv_status tpconv_graph_export(tpconv_graph_t g, int32_t* dst_row_ptr, int32_t* dst_col,
                                  int32_t* dst_eid, int32_t* src_row_ptr, int32_t* src_col,
                                  int32_t* src_eid, hipStream_t stream);

void tpconv_graph_destroy(tpconv_graph_t g);

/* ------------------------------------------------------------- compute --
 * tpconv_forward: out = CGTP convolution of x, Y, W over graph g.
 * One fused kernel: gather of x[src], tensor product and segmented
 * reduction over each destination's CSR row, no per-edge tensor written
 * (FlashTP "Approach": the tensor-product and reduce layers fused into one
 * kernel; its measured-effects table credits this fusion with the larger
 * systems it can hold).  out is overwritten; a node without in-edges gets
 * zeros.  Errors: TPCONV_E_INVALID_ARG (NULL handle or tensor pointer when
 * the tensor is non-empty), TPCONV_E_HIP (launch failure). */
tpconv_status tpconv_forward(tpconv_plan_t plan, tpconv_graph_t g, const void* x, const void* Y,
                             const void* W, void* out, hipStream_t stream);

/* tpconv_backward: gradients of <G, out> for G = grad_out [N][D_out]:
 *   grad_x [N][D_in], grad_Y [E][D_sh], grad_W [E][weight_numel].
 * One fused kernel over the source-sorted CSR: dx is reduced per source
 * row in registers, dY and dW are written once per edge.  Each output is
 * overwritten; pass NULL to skip one (its work is still done when another
 * output needs it).  Errors as tpconv_forward. */
tpconv_status tpconv_backward(tpconv_plan_t plan, tpconv_graph_t g, const void* x, const void* Y,
                              const void* W, const void* grad_out, void* grad_x, void* grad_Y,
                              void* grad_W, hipStream_t stream);

/* tpconv_double_backward: the backward of tpconv_backward -- second
 * derivatives for force-trained potentials (the FlashTP page lists an fp64
 * l_max = 4 double-backward kernel among its key results; the LunaTP and
 * TrimSO(2) abstracts count higher-order derivatives / double backward as
 * part of training).
 * With (dx, dY, dW) = tpconv_backward(x, Y, W, G) and their cotangents
 *   ggx [N][D_in], ggY [E][D_sh], ggW [E][weight_numel]
 * (any may be NULL, meaning zero), it returns the gradients of
 *   L2 = <ggx, dx> + <ggY, dY> + <ggW, dW>
 * with respect to the four inputs:
 *   grad_x [N][D_in], grad_Y [E][D_sh], grad_W [E][weight_numel],
 *   grad_G [N][D_out]  (G = grad_out of the backward).
 * Because the convolution is linear in each input separately, each is the
 * forward or backward with one input replaced by a cotangent, summed:
 *   grad_G = out(ggx, Y, W) + out(x, ggY, W) + out(x, Y, ggW)
 *   grad_x = dx(Y -> ggY) + dx(W -> ggW),  grad_Y = dY(x -> ggx) + dY(W -> ggW),
 *   grad_W = dW(x -> ggx) + dW(Y -> ggY).
 * Two fused kernels: grad_G over the destination-sorted CSR (the forward's
 * structure), the other three over the source-sorted CSR (the backward's).
 * Layouts as tpconv_forward / tpconv_backward.  Each output is overwritten;
 * pass NULL to skip one (grad_G alone skips the second kernel, and the
 * other three alone skip the first).  grad_out may be NULL only when grad_x,
 * grad_Y and grad_W are all NULL.  Errors as tpconv_forward. */
tpconv_status tpconv_double_backward(tpconv_plan_t plan, tpconv_graph_t g, const void* x, const void* Y,
                                     const void* W, const void* grad_out, const void* ggx, const void* ggY,
                                     const void* ggW, void* grad_x, void* grad_Y, void* grad_W, void* grad_G,
                                     hipStream_t stream);

/* ------------------------------------ weights from the radial network --
 * The per-edge weights W [E][weight_numel] are the widest tensor of the
 * layer (the TrimSO(2) abstract names materialised per-edge tensors as the
 * cost to avoid).  In a potential they come from a radial network; its last,
 * linear layer is W = h M, with h [E][hidden] the edges' hidden features
 * (the output of the network's earlier, narrow layers on the edge lengths,
 * computed by the caller) and M [hidden][weight_numel] (columns in W's
 * order; a bias is a constant feature in h).  These two calls take h and M
 * instead of W and generate W inside the kernels, chunk by chunk on the
 * matrix cores into LDS: W is never written to or read from device memory.
 *
 * Supported: fp32 plans whose segments are l = 0..L in order with natural
 * parity on both sides and SH up to L, one multiplicity U in {16, 32, 64},
 * hidden in {16, 32, 64, 128}; h and M device pointers, 16-byte aligned.
 * Other plans or widths: TPCONV_E_UNSUPPORTED (use tpconv_forward /
 * tpconv_backward with W = h M formed by the caller).
 *
 * tpconv_radial_forward: out = tpconv_forward(x, Y, W = h M), overwritten.
 * Errors as tpconv_forward, plus TPCONV_E_UNSUPPORTED as above. */
tpconv_status tpconv_radial_forward(tpconv_plan_t plan, tpconv_graph_t g, int hidden, const void* x,
                                    const void* Y, const void* h, const void* M, void* out, hipStream_t stream);

/* tpconv_radial_backward: gradients of <G, out> for G = grad_out, with
 * W = h M generated in-kernel: grad_x [N][D_in], grad_Y [E][D_sh] and
 * grad_h [E][hidden] = grad_W M^T; and, when grad_W is not NULL, grad_W
 * [E][weight_numel] itself, from which the caller forms the layer's own
 * gradient grad_M = h^T grad_W (training; inference with forces needs only
 * grad_x, grad_Y and grad_h).  Each output is overwritten; NULL skips one.
 * Errors as tpconv_radial_forward. */
tpconv_status tpconv_radial_backward(tpconv_plan_t plan, tpconv_graph_t g, int hidden, const void* x,
                                     const void* Y, const void* h, const void* M, const void* grad_out,
                                     void* grad_x, void* grad_Y, void* grad_h, void* grad_W, hipStream_t stream);

/* ------------------------------------------- upstream: harmonics, forces --
 * The step before the convolution in a force field: the edge harmonics Y
 * from the edge vectors, and the chain rule from grad_Y back to the edge
 * vectors and the atom positions (forces are -dE/dpos).  The LunaTP and
 * TrimSO(2) abstracts place the operator in force-field training; the pages
 * give no formula for this step, which follows from the harmonics'
 * definition.  Separate streaming kernels here; tpconv_forward_vec and
 * tpconv_backward_vec below fuse the same step into the convolution.
 *
 * tpconv_sh: Y[E][(L+1)^2] (L = the plan's sh_lmax, plan dtype) =
 * component-normalised real harmonics of vec[e] / |vec[e]|, (l, m) at column
 * l*l + l + m, the convention of the plan's CG tables (Y_0 = 1,
 * Y_1 = sqrt(3) (y, z, x)).  vec: device [E][3] in the plan's dtype.  A zero
 * vector gets Y = (1, 0, ..., 0).  Errors: TPCONV_E_INVALID_ARG (NULL plan,
 * NULL pointer with n_edges > 0, n_edges < 0), TPCONV_E_HIP. */
tpconv_status tpconv_sh(tpconv_plan_t plan, int64_t n_edges, const void* vec, void* Y, hipStream_t stream);

/* tpconv_sh_backward: grad_vec[E][3] = sum over (l, m) of
 * grad_Y[e][lm] * dY_lm/dvec at vec[e] (zero for a zero vector).  grad_Y
 * [E][(L+1)^2].  Errors as tpconv_sh. */
tpconv_status tpconv_sh_backward(tpconv_plan_t plan, int64_t n_edges, const void* vec, const void* grad_Y,
                                 void* grad_vec, hipStream_t stream);

/* tpconv_positions_backward: grad_pos[N][3] for edge vectors
 * vec[e] = pos[src[e]] - pos[dst[e]] (+ any shift that does not depend on
 * pos): grad_pos[j] = sum of grad_vec over the edges leaving j minus the sum
 * over the edges entering j, over the graph's two CSR views (one wavefront
 * per node, fixed order, deterministic; fp64 sums for fp32 data).
 * grad_vec: [E][3]; grad_pos is overwritten.  Errors as tpconv_sh. */
tpconv_status tpconv_positions_backward(tpconv_plan_t plan, tpconv_graph_t g, const void* grad_vec, void* grad_pos,
                                        hipStream_t stream);

/* The same step inside the convolution kernels ("SH on the fly"): the forward
 * and backward below take the edge vectors instead of Y and evaluate each
 * edge's harmonics themselves (fp64 arithmetic, the values of tpconv_sh), a
 * chunk of a row's edges at a time into on-chip memory; the backward turns
 * each edge's channel-summed dY into grad_vec there.  Y and dY never reach
 * device memory (the LunaTP abstract: reuse across levels of the memory
 * hierarchy; the FlashTP page, "Problem": per-edge intermediates).
 *
 * Supported: every plan of tpconv_forward except those holding both parities
 * of one l (they run as several passes): TPCONV_E_UNSUPPORTED for those (use
 * tpconv_sh, tpconv_forward, tpconv_backward, tpconv_sh_backward).  vec:
 * device [E][3] in the plan's dtype, may be NULL when the graph has no edges.
 *
 * tpconv_forward_vec: out = tpconv_forward(x, tpconv_sh(vec), W), overwritten.
 * Errors as tpconv_forward, plus TPCONV_E_UNSUPPORTED as above. */
tpconv_status tpconv_forward_vec(tpconv_plan_t plan, tpconv_graph_t g, const void* x, const void* vec,
                                 const void* W, void* out, hipStream_t stream);

/* tpconv_backward_vec: gradients of <G, out> for G = grad_out with
 * Y = tpconv_sh(vec): grad_x [N][D_in], grad_W [E][weight_numel] as
 * tpconv_backward, and grad_vec [E][3] = tpconv_sh_backward(vec, grad_Y)
 * in place of grad_Y; tpconv_positions_backward turns grad_vec into forces.
 * Each output is overwritten; NULL skips one.  Errors as tpconv_forward_vec. */
tpconv_status tpconv_backward_vec(tpconv_plan_t plan, tpconv_graph_t g, const void* x, const void* vec,
                                  const void* W, const void* grad_out, void* grad_x, void* grad_vec,
                                  void* grad_W, hipStream_t stream);

/* ------------------------------------------------ SO(2) convolution ------
 * The convolution of SO(2)-based potentials (TrimSO(2), Abstract: rotation
 * on gather, dense matrix multiplications in the edge frame, inverse
 * rotation on reduction; the page prints no formula, so the plainest
 * reading is used).  Per edge e (neighbour j = src, centre i = dst):
 *   x~[l]  = D_e^l x[j, l]                       (per channel)
 *   m = 0: y~_0 = A_0 X_0;   m > 0: y~_+m = A_m X_+m - B_m X_-m,
 *                                   y~_-m = B_m X_+m + A_m X_-m
 *   out[i, l] += D_e^l^T y~[l]
 * X_+-m stacks x~[l][c][+-m] over l = m..L and channels c at index
 * (l - m) C + c; A_m, B_m are shared by all edges.  The output does not
 * depend on the roll of the edge frame about the edge axis.
 *
 * Layouts (row-major, fp32):
 *   x, out, grad  [N][C (L+1)^2]: degree l at column C l^2, stored [C][2l+1]
 *                 (the irreps layout "Cx0e+Cx1o+...", every l = 0..L present)
 *   D             [E][sum_l (2l+1)^2]: block l at sum_{k<l} (2k+1)^2, [m][n]
 *   weights       A_0, A_1, B_1, ..., A_L, B_L, each [K_m][K_m] (out, in),
 *                 K_m = (L+1-m) C; tpconv_so2_weight_numel(L, C) floats.
 * Supported: 1 <= lmax <= 3, channels 16 or 32, TPCONV_F32 (rotations: also
 * lmax 0 and 4, and TPCONV_F64).  Other values: TPCONV_E_UNSUPPORTED. */

/* Number of map weights (and of grad_weights) for (lmax, channels); 0 when
 * the pair is unsupported. */
int64_t tpconv_so2_weight_numel(int lmax, int channels);

/* tpconv_so2_rotations: D[E][sum (2l+1)^2] for edge vectors vec[E][3], both
 * in `dtype`.  The frame R_e is the proper rotation about u x z_hat through
 * the angle between u = vec / |vec| and z_hat (Rodrigues), so R_e u = z_hat;
 * the identity for a zero vector or u = z_hat, diag(1, -1, -1) for
 * u = -z_hat.  D^l(R) is the real Wigner matrix with Y_l(R v) = D^l(R) Y_l(v)
 * for the harmonics of tpconv_sh (fp64 arithmetic inside).  Errors:
 * TPCONV_E_INVALID_ARG (n_edges < 0, NULL pointer with n_edges > 0),
 * TPCONV_E_UNSUPPORTED (lmax outside 0..4), TPCONV_E_HIP. */
tpconv_status tpconv_so2_rotations(int lmax, tpconv_dtype dtype, int64_t n_edges, const void* vec, void* D,
                                   hipStream_t stream);

/* tpconv_so2_forward: out (overwritten, zero rows for nodes without in-edges)
 * over the graph's destination-sorted rows: one block of two wavefronts per
 * row; per chunk of 16 edges the neighbour rows are rotated into an LDS
 * tile, the per-|m| maps run on the matrix cores, and the inverse rotations
 * are summed in registers.  x, D, weights, out: device fp32; weights 16-byte aligned.
 * Errors: TPCONV_E_INVALID_ARG (NULL handle or pointer, misaligned weights),
 * TPCONV_E_UNSUPPORTED, TPCONV_E_HIP. */
tpconv_status tpconv_so2_forward(tpconv_graph_t g, int lmax, int channels, tpconv_dtype dtype, const void* x,
                                 const void* D, const void* weights, void* out, hipStream_t stream);

/* Workspace bytes tpconv_so2_backward needs for n_edges edges: the
 * transposed maps (weight_numel floats) and the partial sums of the map
 * gradients (weight_numel floats per block of edges, at most 512 blocks). */
size_t tpconv_so2_workspace_bytes(int lmax, int channels, int64_t n_edges);

/* tpconv_so2_backward: gradients of <grad_out, out>:
 *   grad_x[j]     = sum_{e: src = j} D_e^T SO2^T(D_e grad_out[dst e])
 *                   (the forward's kernel with the adjoint maps, transposed
 *                   once into the workspace, over the source-sorted rows);
 *   grad_weights  = sum over edges of g~ x~^T per block (g~, x~ the rotated
 *                   grad_out[dst] and x[src]):  A_0: g~_0 X_0^T;
 *                   A_m: g~_+m X_+m^T + g~_-m X_-m^T;
 *                   B_m: g~_-m X_+m^T - g~_+m X_-m^T;
 *                   partial sums per block of edges in `workspace`
 *                   (tpconv_so2_workspace_bytes), then added in block order.
 * Outputs are overwritten; pass NULL to skip one.  The workspace (device,
 * 16-byte aligned, at least tpconv_so2_workspace_bytes) is the caller's and
 * holds nothing between calls.  Deterministic (no atomics).  Errors:
 * TPCONV_E_INVALID_ARG, TPCONV_E_WORKSPACE (workspace too small),
 * TPCONV_E_UNSUPPORTED, TPCONV_E_HIP. */
tpconv_status tpconv_so2_backward(tpconv_graph_t g, int lmax, int channels, tpconv_dtype dtype, const void* x,
                                  const void* D, const void* weights, const void* grad_out, void* grad_x,
                                  void* grad_weights, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* tpconv_so2_backward_noalloc: tpconv_so2_backward without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).  It
 * allocates nothing: the transposed maps and the partial map gradients live
 * in a 16 MiB device array of the library (one per device, held until the
 * process ends; every l <= 3, C <= 32 map set fits, with at least 92 blocks
 * of edges).  Same arguments, outputs, results and errors as
 * tpconv_so2_backward; grad_x is bitwise the same, grad_weights may sum its
 * blocks of edges differently (fewer blocks when the scratch is the limit).
 * Maps larger than the scratch get TPCONV_E_WORKSPACE.  The scratch keeps the
 * last call's contents and holds nothing a call needs at its start; calls
 * that overlap on one device (two streams, or host threads) race on it and
 * must be ordered by the caller. */
tpconv_status tpconv_so2_backward_noalloc(tpconv_graph_t g, int lmax, int channels, tpconv_dtype dtype,
                                          const void* x, const void* D, const void* weights, const void* grad_out,
                                          void* grad_x, void* grad_weights, hipStream_t stream);

/* tpconv_so2_double_backward: the backward of tpconv_so2_backward, with the
 * frames D held fixed (the TrimSO(2) abstract counts the double backward
 * among the operator's passes).  With (grad_x, grad_w) = the backward of
 * (x, weights, grad_out) and their cotangents ggx [N][C (L+1)^2] and
 * ggw [weight_numel] (either may be NULL = zero), it returns the gradients
 * of L2 = <ggx, grad_x> + <ggw, grad_w>.  The convolution f(x; w) is linear
 * in x and in w separately, so
 *   grad_G       = f(ggx; w) + f(x; ggw)          [N][C (L+1)^2]
 *   grad_x       = f(.; ggw)^T grad_out           (the backward's grad_x, ggw for w)
 *   grad_weights = map gradient of (ggx, grad_out) (the backward's grad_w, ggx for x)
 * each from the same kernels as the forward and backward (the second
 * forward adds into grad_G; each row has one writer).  Outputs are
 * overwritten; pass NULL to skip one.  Workspace and alignment as
 * tpconv_so2_backward (needed when grad_x or grad_weights is asked for; ggw
 * 16-byte aligned).  Errors as tpconv_so2_backward. */
tpconv_status tpconv_so2_double_backward(tpconv_graph_t g, int lmax, int channels, tpconv_dtype dtype, const void* x,
                                         const void* D, const void* weights, const void* grad_out, const void* ggx,
                                         const void* ggw, void* grad_x, void* grad_weights, void* grad_G,
                                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* tpconv_so2_frames_backward: grad_D [E][sum (2l+1)^2] (overwritten), the
 * gradient of <grad_out, out> with respect to each edge's Wigner blocks, for
 * forces through the edge frames (chain on with tpconv_so2_rotations_backward
 * and tpconv_positions_backward).  D_e enters twice, so with
 * x~ = D_e x[src], y~ = SO2(x~), dx~ = SO2^T(D_e grad_out[dst]):
 *   grad_D[e]^l[m][n] = sum_c y~[l][c][m] grad_out[dst][l][c][n]
 *                     + sum_c dx~[l][c][m] x[src][l][c][n].
 * The forward's kernel recomputes y~ over the destination rows and the
 * adjoint's recomputes dx~ over the source rows (no per-edge tensor is
 * kept between passes); each contracts its tile with the row's own vector.
 * Workspace, alignment and errors as tpconv_so2_backward. */
tpconv_status tpconv_so2_frames_backward(tpconv_graph_t g, int lmax, int channels, tpconv_dtype dtype, const void* x,
                                         const void* D, const void* weights, const void* grad_out, void* grad_D,
                                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* tpconv_so2_rotations_backward: grad_vec [E][3] (overwritten) =
 * sum over blocks of grad_D[e] . dD/dvec for D = tpconv_so2_rotations(vec),
 * differentiating the same quadrature through the frame (dual numbers,
 * fp64 inside).  Vectors on the z axis (and the zero vector), where the
 * frame is a convention, get zero.  Errors as tpconv_so2_rotations. */
tpconv_status tpconv_so2_rotations_backward(int lmax, tpconv_dtype dtype, int64_t n_edges, const void* vec,
                                            const void* grad_D, void* grad_vec, hipStream_t stream);

/* tpconv_so2_rotations_jvp: dD [E][sum (2l+1)^2] (overwritten), the
 * directional derivative of tpconv_so2_rotations(vec) along dvec [E][3]
 * per edge -- the same dual numbers as tpconv_so2_rotations_backward,
 * contracted with dvec.  With dvec the cotangent of the edge-vector gradient
 * (e.g. of forces), dD is the cotangent that
 * tpconv_so2_frames_double_backward takes.  Vectors on the z axis (and the
 * zero vector) get zero.  Errors as tpconv_so2_rotations. */
tpconv_status tpconv_so2_rotations_jvp(int lmax, tpconv_dtype dtype, int64_t n_edges, const void* vec,
                                       const void* dvec, void* dD, hipStream_t stream);

/* tpconv_so2_frames_double_backward: the mixed second derivatives through
 * the edge frames that training on forces needs (the TrimSO(2) abstract asks
 * for the higher-order differentiation of training).  With grad_D =
 * tpconv_so2_frames_backward(x, D, weights, grad_out) and a cotangent dD of
 * the same shape, it returns the gradients of S = <dD, grad_D> with respect
 * to x, the weights and grad_out (frames D held fixed):
 *   grad_G[dst]  += dD_e^T SO2(D_e x) + D_e^T SO2(dD_e x)
 *   grad_x[src]  += D_e^T SO2^T(dD_e g) + dD_e^T SO2^T(D_e g)
 *   grad_weights  = the map gradients of (dD_e g, D_e x) and (D_e g, dD_e x)
 * (g = grad_out[dst], x = x[src]): each term one pass of the forward, the
 * adjoint or the map-gradient kernel with different blocks in its two
 * rotation places (the second of each pair adds into the first's output;
 * each row has one writer).  dD is first replaced, per edge, by dD minus its
 * least-squares component along J D (J the generator of rolls about the edge
 * axis), in fp64: the convolution does not change when an edge's frame rolls
 * about its axis, so this changes no result in exact arithmetic, and it
 * removes the roll rate of a frames' derivative, which is unbounded for
 * edges near the frames' pole and whose two terms cancel in fp32.  Outputs (grad_x, grad_G [N][C (L+1)^2],
 * grad_weights [weight_numel]) are overwritten; NULL skips one.  workspace:
 * at least tpconv_so2_frames_double_backward_workspace_bytes(...), 256-byte
 * aligned, caller-owned; weights 16-byte aligned.  Errors:
 * TPCONV_E_INVALID_ARG, TPCONV_E_UNSUPPORTED (as tpconv_so2_forward),
 * TPCONV_E_WORKSPACE, TPCONV_E_HIP. */
size_t tpconv_so2_frames_double_backward_workspace_bytes(int lmax, int channels, int64_t n_nodes, int64_t n_edges);
tpconv_status tpconv_so2_frames_double_backward(tpconv_graph_t g, int lmax, int channels, tpconv_dtype dtype,
                                                const void* x, const void* D, const void* weights,
                                                const void* grad_out, const void* dD, void* grad_x,
                                                void* grad_weights, void* grad_G, void* workspace,
                                                size_t workspace_bytes, hipStream_t stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* tpconv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TPCONV_H */
