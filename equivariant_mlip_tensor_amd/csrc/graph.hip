// graph.hip -- destination- and source-sorted CSR views of an edge list.
//
// The convolution runs node-centric (LunaTP Abstract): the forward walks
// each destination's in-edges, the backward each source's out-edges, so
// both reductions happen in registers of one wavefront.  The layout is a
// counting sort done on the device -- histogram, scan, scatter -- followed by
// a per-row sort on the edge id (one wavefront per row ranks each edge by
// the number of the row's edges with a smaller id), so every row lists its
// edges in the caller's order and the layout (and every sum over a row) is
// deterministic.
// Each view also gets a row order, longest rows first, in which the kernels
// hand rows to wavefronts: the long rows start early and the short ones fill
// the tail of the dispatch.  Rows of equal degree may come in any order; a
// row's result does not depend on when it runs.  Integer atomics are used
// only here, to count and place edges and rows.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <new>
#include <string>

#include "tpconv_internal.hpp"

namespace tpconv {
namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Rows are handed to wavefronts longest first: bucket of a row = min(degree,
// kDegBuckets - 1), buckets visited from the highest degree down.
constexpr int kDegBuckets = 1024;

struct Layout {
  size_t dst_row, dst_col, dst_eid, src_row, src_col, src_eid, dst_order, src_order, cur_dst, cur_src, hist,
      hcur, err, tmp_dcol, tmp_deid, tmp_scol, tmp_seid, total;
};

Layout layout(int64_t n, int64_t e) {
  Layout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  L.dst_row = take(sizeof(int32_t) * (n + 1));
  L.dst_col = take(sizeof(int32_t) * e);
  L.dst_eid = take(sizeof(int32_t) * e);
  L.src_row = take(sizeof(int32_t) * (n + 1));
  L.src_col = take(sizeof(int32_t) * e);
  L.src_eid = take(sizeof(int32_t) * e);
  L.dst_order = take(sizeof(int32_t) * n);
  L.src_order = take(sizeof(int32_t) * n);
  L.cur_dst = take(sizeof(int32_t) * n);
  L.cur_src = take(sizeof(int32_t) * n);
  L.hist = take(sizeof(int32_t) * 2 * kDegBuckets);
  L.hcur = take(sizeof(int32_t) * 2 * kDegBuckets);
  L.err = take(sizeof(int32_t));
  // the scatter's unsorted rows, read once by the per-row sort
  L.tmp_dcol = take(sizeof(int32_t) * e);
  L.tmp_deid = take(sizeof(int32_t) * e);
  L.tmp_scol = take(sizeof(int32_t) * e);
  L.tmp_seid = take(sizeof(int32_t) * e);
  L.total = o;
  return L;
}

__global__ void k_fill(int32_t* __restrict__ p, int64_t n, int32_t v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

__global__ void k_count(const int32_t* __restrict__ src, const int32_t* __restrict__ dst, int64_t E, int64_t N,
                        int32_t* __restrict__ dst_cnt, int32_t* __restrict__ src_cnt, int32_t* __restrict__ err) {
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < E; e += (int64_t)gridDim.x * blockDim.x) {
    const int32_t s = src[e], d = dst[e];
    if (s < 0 || s >= N || d < 0 || d >= N) {
      atomicAdd(err, 1);
      continue;
    }
    atomicAdd(&dst_cnt[d], 1);
    atomicAdd(&src_cnt[s], 1);
  }
}

// In-place inclusive scan of p[0..n) by one 1024-thread block: each thread
// sums a contiguous run, the run totals are scanned in LDS, then each run is
// rewritten with its offset.
__global__ __launch_bounds__(1024) void k_scan(int32_t* __restrict__ p, int64_t n) {
  __shared__ int32_t part[1024];
  const int t = threadIdx.x;
  const int64_t per = (n + 1023) / 1024;
  const int64_t a = t * per;
  const int64_t b = a + per < n ? a + per : n;
  int32_t s = 0;
  for (int64_t i = a; i < b; ++i) s += p[i];
  part[t] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int32_t run = t > 0 ? part[t - 1] : 0;
  for (int64_t i = a; i < b; ++i) {
    run += p[i];
    p[i] = run;
  }
}

__global__ void k_scatter(const int32_t* __restrict__ src, const int32_t* __restrict__ dst, int64_t E, int64_t N,
                          const int32_t* __restrict__ dst_row, int32_t* __restrict__ cur_dst,
                          int32_t* __restrict__ dst_col, int32_t* __restrict__ dst_eid,
                          const int32_t* __restrict__ src_row, int32_t* __restrict__ cur_src,
                          int32_t* __restrict__ src_col, int32_t* __restrict__ src_eid) {
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < E; e += (int64_t)gridDim.x * blockDim.x) {
    const int32_t s = src[e], d = dst[e];
    if (s < 0 || s >= N || d < 0 || d >= N) continue;
    const int32_t pd = dst_row[d] + atomicAdd(&cur_dst[d], 1);
    dst_col[pd] = s;
    dst_eid[pd] = static_cast<int32_t>(e);
    const int32_t ps = src_row[s] + atomicAdd(&cur_src[s], 1);
    src_col[ps] = d;
    src_eid[ps] = static_cast<int32_t>(e);
  }
}

// One wavefront per row: each of the row's (eid, col) pairs goes to the
// position given by the number of the row's edges with a smaller eid (eids
// in a row are distinct, so these ranks are a permutation).  Lanes take the
// row 64 edges at a time and compare against it 64 at a time through lane
// shuffles; the loop bounds are the same for the whole wave.
__global__ __launch_bounds__(256) void k_rank_rows(const int32_t* __restrict__ row, const int32_t* __restrict__ col_in,
                                                   const int32_t* __restrict__ eid_in, int32_t* __restrict__ col_out,
                                                   int32_t* __restrict__ eid_out, int64_t N) {
  const int lane = threadIdx.x & 63;
  for (int64_t r = blockIdx.x * 4 + (threadIdx.x >> 6); r < N; r += (int64_t)gridDim.x * 4) {
    const int32_t a = row[r];
    const int32_t d = row[r + 1] - a;
    for (int32_t base = 0; base < d; base += 64) {
      const int32_t i = base + lane;
      const bool mine = i < d;
      const int32_t me = mine ? eid_in[a + i] : 0;
      const int32_t mc = mine ? col_in[a + i] : 0;
      int32_t rank = 0;
      for (int32_t cb = 0; cb < d; cb += 64) {
        const int32_t j = cb + lane;
        const int32_t other = j < d ? eid_in[a + j] : 0;
        const int32_t lim = d - cb < 64 ? d - cb : 64;
        for (int32_t k = 0; k < lim; ++k) rank += __shfl(other, k, 64) < me ? 1 : 0;
      }
      if (mine) {
        eid_out[a + rank] = me;
        col_out[a + rank] = mc;
      }
    }
  }
}

__device__ __forceinline__ int deg_bucket(const int32_t* row, int64_t r) {
  const int d = row[r + 1] - row[r];
  const int b = d < kDegBuckets - 1 ? d : kDegBuckets - 1;
  return kDegBuckets - 1 - b;  // bucket 0 holds the longest rows
}

__global__ void k_deg_hist(const int32_t* __restrict__ row, int64_t N, int32_t* __restrict__ hist) {
  for (int64_t r = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; r < N; r += (int64_t)gridDim.x * blockDim.x)
    atomicAdd(&hist[deg_bucket(row, r)], 1);
}

// hist holds inclusive bucket ends after k_scan; order[] lists rows longest first
__global__ void k_deg_order(const int32_t* __restrict__ row, int64_t N, const int32_t* __restrict__ hist,
                            int32_t* __restrict__ hcur, int32_t* __restrict__ order) {
  for (int64_t r = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; r < N; r += (int64_t)gridDim.x * blockDim.x) {
    const int b = deg_bucket(row, r);
    const int32_t start = b > 0 ? hist[b - 1] : 0;
    order[start + atomicAdd(&hcur[b], 1)] = static_cast<int32_t>(r);
  }
}

int grid_for(int64_t n, int block) {
  int64_t g = (n + block - 1) / block;
  if (g < 1) g = 1;
  if (g > 65536) g = 65536;
  return static_cast<int>(g);
}

}  // namespace
}  // namespace tpconv

using tpconv::fail;
using tpconv::Graph;

extern "C" size_t tpconv_graph_workspace_bytes(int64_t n_nodes, int64_t n_edges) {
  if (n_nodes < 0 || n_edges < 0) return 0;
  return tpconv::layout(n_nodes, n_edges).total;
}

extern "C" tpconv_status tpconv_graph_create(int64_t n_nodes, int64_t n_edges, const int32_t* src,
                                             const int32_t* dst, void* workspace, size_t workspace_bytes,
                                             hipStream_t stream, tpconv_graph_t* out) {
  using namespace tpconv;
  if (out == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL output handle");
  *out = nullptr;
  if (n_nodes < 0 || n_edges < 0) return fail(TPCONV_E_INVALID_ARG, "negative node or edge count");
  if (n_edges >= INT32_MAX || n_nodes >= INT32_MAX)
    return fail(TPCONV_E_INVALID_ARG, "node and edge counts must be below 2^31");
  if (n_edges > 0 && (src == nullptr || dst == nullptr)) return fail(TPCONV_E_INVALID_ARG, "NULL src or dst");
  if (workspace == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL workspace");
  const Layout L = layout(n_nodes, n_edges);
  if (workspace_bytes < L.total)
    return fail(TPCONV_E_WORKSPACE, "workspace holds " + std::to_string(workspace_bytes) + " bytes, needs " +
                                         std::to_string(L.total));
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
    return fail(TPCONV_E_WORKSPACE, "workspace must be 256-byte aligned");

  char* base = static_cast<char*>(workspace);
  auto at = [&](size_t off) { return reinterpret_cast<int32_t*>(base + off); };
  Graph g;
  g.n_nodes = n_nodes;
  g.n_edges = n_edges;
  g.dst_row = at(L.dst_row);
  g.dst_col = at(L.dst_col);
  g.dst_eid = at(L.dst_eid);
  g.src_row = at(L.src_row);
  g.src_col = at(L.src_col);
  g.src_eid = at(L.src_eid);
  g.dst_order = at(L.dst_order);
  g.src_order = at(L.src_order);
  int32_t* hist = at(L.hist);
  int32_t* hcur = at(L.hcur);
  int32_t* cur_dst = at(L.cur_dst);
  int32_t* cur_src = at(L.cur_src);
  int32_t* err = at(L.err);
  int32_t* tmp_dcol = at(L.tmp_dcol);
  int32_t* tmp_deid = at(L.tmp_deid);
  int32_t* tmp_scol = at(L.tmp_scol);
  int32_t* tmp_seid = at(L.tmp_seid);

  const int B = 256;
  hipLaunchKernelGGL(k_fill, dim3(grid_for(n_nodes + 1, B)), dim3(B), 0, stream, g.dst_row, n_nodes + 1, 0);
  hipLaunchKernelGGL(k_fill, dim3(grid_for(n_nodes + 1, B)), dim3(B), 0, stream, g.src_row, n_nodes + 1, 0);
  if (n_nodes > 0) {
    hipLaunchKernelGGL(k_fill, dim3(grid_for(n_nodes, B)), dim3(B), 0, stream, cur_dst, n_nodes, 0);
    hipLaunchKernelGGL(k_fill, dim3(grid_for(n_nodes, B)), dim3(B), 0, stream, cur_src, n_nodes, 0);
  }
  hipLaunchKernelGGL(k_fill, dim3(1), dim3(B), 0, stream, err, int64_t(1), 0);
  hipLaunchKernelGGL(k_fill, dim3(grid_for(4 * kDegBuckets, B)), dim3(B), 0, stream, hist, int64_t(2 * kDegBuckets), 0);
  hipLaunchKernelGGL(k_fill, dim3(grid_for(4 * kDegBuckets, B)), dim3(B), 0, stream, hcur, int64_t(2 * kDegBuckets), 0);
  if (n_edges > 0) {
    hipLaunchKernelGGL(k_count, dim3(grid_for(n_edges, B)), dim3(B), 0, stream, src, dst, n_edges, n_nodes,
                       g.dst_row + 1, g.src_row + 1, err);
  }
  if (n_nodes > 0) {
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, stream, g.dst_row + 1, n_nodes);
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, stream, g.src_row + 1, n_nodes);
  }
  if (n_edges > 0) {
    hipLaunchKernelGGL(k_scatter, dim3(grid_for(n_edges, B)), dim3(B), 0, stream, src, dst, n_edges, n_nodes,
                       g.dst_row, cur_dst, tmp_dcol, tmp_deid, g.src_row, cur_src, tmp_scol, tmp_seid);
    hipLaunchKernelGGL(k_rank_rows, dim3(grid_for((n_nodes + 3) / 4, 1)), dim3(256), 0, stream, g.dst_row, tmp_dcol,
                       tmp_deid, g.dst_col, g.dst_eid, n_nodes);
    hipLaunchKernelGGL(k_rank_rows, dim3(grid_for((n_nodes + 3) / 4, 1)), dim3(256), 0, stream, g.src_row, tmp_scol,
                       tmp_seid, g.src_col, g.src_eid, n_nodes);
  }
  if (n_nodes > 0) {
    const int32_t* rows[2] = {g.dst_row, g.src_row};
    int32_t* orders[2] = {g.dst_order, g.src_order};
    for (int v = 0; v < 2; ++v) {
      int32_t* h = hist + v * kDegBuckets;
      hipLaunchKernelGGL(k_deg_hist, dim3(grid_for(n_nodes, B)), dim3(B), 0, stream, rows[v], n_nodes, h);
      hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, stream, h, int64_t(kDegBuckets));
      hipLaunchKernelGGL(k_deg_order, dim3(grid_for(n_nodes, B)), dim3(B), 0, stream, rows[v], n_nodes, h,
                         hcur + v * kDegBuckets, orders[v]);
    }
  }
  hipError_t he = hipGetLastError();
  if (he != hipSuccess) return fail(TPCONV_E_HIP, std::string("graph build launch: ") + hipGetErrorString(he));
  int32_t h_err = 0;
  he = hipMemcpyAsync(&h_err, err, sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (he == hipSuccess) he = hipStreamSynchronize(stream);
  if (he != hipSuccess) return fail(TPCONV_E_HIP, std::string("graph build: ") + hipGetErrorString(he));
  if (h_err > 0)
    return fail(TPCONV_E_INDEX, std::to_string(h_err) + " edge(s) have src or dst outside [0, " +
                                    std::to_string(n_nodes) + ")");
  Graph* h = new (std::nothrow) Graph(g);
  if (h == nullptr) return fail(TPCONV_E_INVALID_ARG, "out of host memory");
  *out = reinterpret_cast<tpconv_graph_t>(h);
  return TPCONV_OK;
}

extern "C" tpconv_status tpconv_graph_export(tpconv_graph_t hg, int32_t* dst_row_ptr, int32_t* dst_col,
                                             int32_t* dst_eid, int32_t* src_row_ptr, int32_t* src_col,
                                             int32_t* src_eid, hipStream_t stream) {
  if (hg == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL graph");
  const Graph& g = *reinterpret_cast<const Graph*>(hg);
  struct Item {
    int32_t* host;
    const int32_t* dev;
    int64_t n;
  } items[] = {{dst_row_ptr, g.dst_row, g.n_nodes + 1}, {dst_col, g.dst_col, g.n_edges},
               {dst_eid, g.dst_eid, g.n_edges},         {src_row_ptr, g.src_row, g.n_nodes + 1},
               {src_col, g.src_col, g.n_edges},         {src_eid, g.src_eid, g.n_edges}};
  for (const Item& it : items) {
    if (it.host == nullptr || it.n == 0) continue;
    const hipError_t he =
        hipMemcpyAsync(it.host, it.dev, sizeof(int32_t) * it.n, hipMemcpyDeviceToHost, stream);
    if (he != hipSuccess) return fail(TPCONV_E_HIP, std::string("graph export: ") + hipGetErrorString(he));
  }
  const hipError_t he = hipStreamSynchronize(stream);
  if (he != hipSuccess) return fail(TPCONV_E_HIP, std::string("graph export: ") + hipGetErrorString(he));
  return TPCONV_OK;
}

extern "C" void tpconv_graph_destroy(tpconv_graph_t g) { delete reinterpret_cast<Graph*>(g); }
