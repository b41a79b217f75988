// graph.hip -- destination- and source-sorted CSR views of an edge list.
//
// The convolution runs node-centric (LunaTP Abstract): the forward walks
// each destination's in-edges, the backward each source's out-edges, so
// both reductions happen in registers of one wavefront.  Each view is a
// stable radix sort of the edge ids by destination (resp. source) node
// (rocPRIM), so every row lists its edges in the caller's order and the
// layout (and every sum over a row) is deterministic; each row pointer is a
// binary search of the sorted node ids.  Nothing counts with atomics, so the
// cost is linear in the edge count whatever the degree distribution (a hub
// row of 10^5 edges costs what 10^5 edges spread over many rows cost).
// Each view also gets a row order, longest rows first (a stable radix sort
// of the rows by degree, capped at kDegBuckets - 1), in which the kernels
// hand rows to wavefronts: the long rows start early and the short ones fill
// the tail of the dispatch.  The only atomic counts edges with an index out
// of range.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <new>
#include <string>

#include <rocprim/device/device_radix_sort.hpp>
#include <rocprim/iterator/counting_iterator.hpp>

#include "tpconv_internal.hpp"

namespace tpconv {
namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Rows are handed to wavefronts longest first: sort key of a row =
// kDegBuckets - 1 - min(degree, kDegBuckets - 1), ascending.
constexpr int kDegBuckets = 1024;
constexpr unsigned kDegBits = 10;

struct Layout {
  size_t dst_row, dst_col, dst_eid, src_row, src_col, src_eid, dst_order, src_order, dkey, dkey_out, err, keys,
      temp, total;
};

// Scratch of the library sort of n keys (a host-side size query; nothing runs).
size_t sort_temp_bytes(int64_t n) {
  size_t bytes = 0;
  (void)rocprim::radix_sort_pairs(nullptr, bytes, static_cast<const int32_t*>(nullptr), static_cast<int32_t*>(nullptr),
                                  rocprim::counting_iterator<int32_t>(0), static_cast<int32_t*>(nullptr),
                                  static_cast<int32_t>(n), 0u, 32u, hipStream_t(0));
  return bytes;
}

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
  L.dkey = take(sizeof(int32_t) * n);      // rows' degree keys and their sorted copy (not kept)
  L.dkey_out = take(sizeof(int32_t) * n);
  L.err = take(sizeof(int32_t));
  L.keys = take(sizeof(int32_t) * e);      // the edge sorts' key output (not kept)
  L.temp = take(std::max({e > 0 ? sort_temp_bytes(e) : size_t(0), n > 0 ? sort_temp_bytes(n) : size_t(0),
                          size_t(1)}));
  L.total = o;
  return L;
}

__global__ void k_fill(int32_t* __restrict__ p, int64_t n, int32_t v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// Counts edges with an end outside [0, N).
__global__ void k_check(const int32_t* __restrict__ src, const int32_t* __restrict__ dst, int64_t E, int64_t N,
                        int32_t* __restrict__ err) {
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < E; e += (int64_t)gridDim.x * blockDim.x) {
    const int32_t s = src[e], d = dst[e];
    if (s < 0 || s >= N || d < 0 || d >= N) atomicAdd(err, 1);
  }
}

// row[k] = first position of the sorted node ids holding k or more (k = 0..N)
__global__ void k_row_bounds(const int32_t* __restrict__ keys, int64_t E, int64_t N, int32_t* __restrict__ row) {
  for (int64_t k = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; k <= N; k += (int64_t)gridDim.x * blockDim.x) {
    int64_t lo = 0, hi = E;
    while (lo < hi) {
      const int64_t mid = (lo + hi) >> 1;
      if (keys[mid] < k)
        lo = mid + 1;
      else
        hi = mid;
    }
    row[k] = static_cast<int32_t>(lo);
  }
}

// col[i] = other end of the edge at position i of a view
__global__ void k_gather_col(const int32_t* __restrict__ eid, const int32_t* __restrict__ other, int64_t E,
                             int32_t* __restrict__ col) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < E; i += (int64_t)gridDim.x * blockDim.x)
    col[i] = other[eid[i]];
}

// sort key of each row: longest rows get the smallest key
__global__ void k_deg_key(const int32_t* __restrict__ row, int64_t N, int32_t* __restrict__ key) {
  for (int64_t r = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; r < N; r += (int64_t)gridDim.x * blockDim.x) {
    const int d = row[r + 1] - row[r];
    key[r] = kDegBuckets - 1 - (d < kDegBuckets - 1 ? d : kDegBuckets - 1);
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
  int32_t* dkey = at(L.dkey);
  int32_t* dkey_out = at(L.dkey_out);
  int32_t* err = at(L.err);
  int32_t* keys = at(L.keys);
  void* temp = base + L.temp;

  const int B = 256;
  hipLaunchKernelGGL(k_fill, dim3(1), dim3(B), 0, stream, err, int64_t(1), 0);
  hipError_t he = hipSuccess;
  auto check = [&](hipError_t e, const char* what) {
    if (he == hipSuccess && e != hipSuccess) {
      he = e;
      return fail(TPCONV_E_HIP, std::string("graph build (") + what + "): " + hipGetErrorString(e));
    }
    return TPCONV_OK;
  };
  if (n_edges > 0)
    hipLaunchKernelGGL(k_check, dim3(grid_for(n_edges, B)), dim3(B), 0, stream, src, dst, n_edges, n_nodes, err);
  // stable sorts of the edge ids by node (keys are node ids < n_nodes; an
  // out-of-range id is reported below and the graph discarded), then the row
  // pointers by binary search of the sorted ids
  const unsigned bits =
      n_nodes > 1 ? 32u - static_cast<unsigned>(__builtin_clz(static_cast<uint32_t>(n_nodes - 1))) : 1u;
  const int32_t* key_in[2] = {dst, src};
  const int32_t* other[2] = {src, dst};
  int32_t* eid_out[2] = {g.dst_eid, g.src_eid};
  int32_t* col_out[2] = {g.dst_col, g.src_col};
  int32_t* rows[2] = {g.dst_row, g.src_row};
  int32_t* orders[2] = {g.dst_order, g.src_order};
  for (int v = 0; v < 2; ++v) {
    if (n_edges > 0) {
      size_t tb = L.total - L.temp;
      const tpconv_status st =
          check(rocprim::radix_sort_pairs(temp, tb, key_in[v], keys, rocprim::counting_iterator<int32_t>(0),
                                          eid_out[v], static_cast<int32_t>(n_edges), 0u, bits, stream),
                "edge sort");
      if (st != TPCONV_OK) return st;
      hipLaunchKernelGGL(k_gather_col, dim3(grid_for(n_edges, B)), dim3(B), 0, stream, eid_out[v], other[v], n_edges,
                         col_out[v]);
    }
    hipLaunchKernelGGL(k_row_bounds, dim3(grid_for(n_nodes + 1, B)), dim3(B), 0, stream, keys, n_edges, n_nodes,
                       rows[v]);
    if (n_nodes > 0) {
      hipLaunchKernelGGL(k_deg_key, dim3(grid_for(n_nodes, B)), dim3(B), 0, stream, rows[v], n_nodes, dkey);
      size_t tb = L.total - L.temp;
      const tpconv_status st =
          check(rocprim::radix_sort_pairs(temp, tb, dkey, dkey_out, rocprim::counting_iterator<int32_t>(0), orders[v],
                                          static_cast<int32_t>(n_nodes), 0u, kDegBits, stream),
                "row order");
      if (st != TPCONV_OK) return st;
    }
  }
  he = hipGetLastError();
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
