// tpconv_internal.hpp -- host-side structs behind the opaque C handles.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "tp_common.hpp"
#include "tpconv.h"

namespace tpconv {

struct Segment {
  int mul;
  int l;
  int p;  // +1 even, -1 odd
};

struct Path {
  int s1, l2, s3;
  int64_t woff;  // first W column of the path
};

// One launch's share of a plan that holds both parities of some l: the
// input segments of one type t_in and the output segments of one type t_out,
// where a segment's type is p (-1)^l (+1 natural, -1 the other), and the
// plan's paths between them (even l1 + l2 + l3 when the types agree, odd
// otherwise).  Each l appears at most once on either side of a pass.
struct Pass {
  int t_in = 1, t_out = 1;
  int32_t in_off[kMaxL + 1];
  int32_t out_off[kMaxL + 1];
  int32_t woff[kMaxTriples];
  uint64_t pmask_lo = 0, pmask_hi = 0;
  int n_in = 0, n_out = 0, n_paths = 0;  // segments and paths in the pass
};

struct Plan {
  std::vector<Segment> in, out;
  int sh_lmax = 0;
  tpconv_dtype dtype = TPCONV_F32;
  int mul = 0;
  int kernel_l = 0;
  int64_t dim_in = 0, dim_out = 0, dim_sh = 0;
  std::vector<Path> paths;
  int64_t weight_numel = 0;
  // sparse real CG table
  std::vector<uint32_t> entries;
  std::vector<int32_t> path_ptr;
  std::vector<double> values;
  // kernel arguments fixed by the plan
  int32_t in_off[kMaxL + 1];
  int32_t out_off[kMaxL + 1];
  int32_t woff[kMaxTriples];
  uint64_t pmask_lo = 0, pmask_hi = 0;
  // plans with both parities of some l run as up to four passes (empty for
  // the others, which run as one launch with the fields above)
  std::vector<Pass> passes;

  static tpconv_status build(const char* irreps_in, int sh_lmax, const char* irreps_out, tpconv_dtype dt,
                             Plan& p);
};

struct Graph {
  int64_t n_nodes = 0, n_edges = 0;
  // destination-sorted CSR: row i lists edges with dst == i; col = src
  int32_t* dst_row = nullptr;
  int32_t* dst_col = nullptr;
  int32_t* dst_eid = nullptr;
  // source-sorted CSR: row j lists edges with src == j; col = dst
  int32_t* src_row = nullptr;
  int32_t* src_col = nullptr;
  int32_t* src_eid = nullptr;
  // rows of each view sorted by decreasing degree (scheduling order)
  int32_t* dst_order = nullptr;
  int32_t* src_order = nullptr;
};

// Records the message for tpconv_last_error() and returns the status.
tpconv_status fail(tpconv_status st, const std::string& msg);

}  // namespace tpconv
