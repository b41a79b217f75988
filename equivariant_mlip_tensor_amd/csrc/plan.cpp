// plan.cpp -- irreps parsing, path enumeration and the sparse CG table (host).
//
// The plan is the host-side half of the convolution: it parses the irreps,
// lists the admissible paths in lexicographic (s1, l2, s3) order -- the
// column order of W -- and emits the sparse real CG matrix as COO with
// deduplicated values (FlashTP "Approach").  Consecutive paths share their
// (s1, l2) input, which is the grouping the kernels exploit to form each
// x (x) Y product once per group.
#include <algorithm>
#include <cctype>
#include <cmath>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "tpconv.h"
#include "tpconv_internal.hpp"

namespace tpconv {

namespace {

bool parse_irreps(const char* text, std::vector<Segment>& out, std::string& why) {
  out.clear();
  if (text == nullptr) {
    why = "irreps string is NULL";
    return false;
  }
  const std::string s(text);
  size_t i = 0;
  auto skip_ws = [&]() {
    while (i < s.size() && std::isspace(static_cast<unsigned char>(s[i]))) ++i;
  };
  auto read_int = [&](long& v) -> bool {
    if (i >= s.size() || !std::isdigit(static_cast<unsigned char>(s[i]))) return false;
    v = 0;
    while (i < s.size() && std::isdigit(static_cast<unsigned char>(s[i]))) {
      v = v * 10 + (s[i] - '0');
      if (v > (1L << 30)) return false;
      ++i;
    }
    return true;
  };
  for (;;) {
    skip_ws();
    long a = 0;
    if (!read_int(a)) {
      why = "expected a number at position " + std::to_string(i) + " of '" + s + "'";
      return false;
    }
    skip_ws();
    long mul = 1, l = a;
    if (i < s.size() && s[i] == 'x') {
      ++i;
      skip_ws();
      mul = a;
      if (!read_int(l)) {
        why = "expected l after 'x' at position " + std::to_string(i) + " of '" + s + "'";
        return false;
      }
      skip_ws();
    }
    if (i >= s.size() || (s[i] != 'e' && s[i] != 'o')) {
      why = "expected parity 'e' or 'o' at position " + std::to_string(i) + " of '" + s + "'";
      return false;
    }
    const int p = s[i] == 'e' ? 1 : -1;
    ++i;
    if (mul <= 0) {
      why = "multiplicity must be positive in '" + s + "'";
      return false;
    }
    out.push_back(Segment{static_cast<int>(mul), static_cast<int>(l), p});
    skip_ws();
    if (i == s.size()) break;
    if (s[i] != '+') {
      why = "expected '+' at position " + std::to_string(i) + " of '" + s + "'";
      return false;
    }
    ++i;
  }
  return true;
}

}  // namespace

tpconv_status Plan::build(const char* irreps_in, int sh_lmax_, const char* irreps_out, tpconv_dtype dt,
                          Plan& p) {
  if (irreps_in == nullptr || irreps_out == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL irreps string");
  if (sh_lmax_ < 0) return fail(TPCONV_E_INVALID_ARG, "sh_lmax must be >= 0");
  if (dt != TPCONV_F32 && dt != TPCONV_F64) return fail(TPCONV_E_INVALID_ARG, "dtype must be TPCONV_F32 or TPCONV_F64");
  std::string why;
  if (!parse_irreps(irreps_in, p.in, why)) return fail(TPCONV_E_IRREPS, "irreps_in: " + why);
  if (!parse_irreps(irreps_out, p.out, why)) return fail(TPCONV_E_IRREPS, "irreps_out: " + why);
  p.sh_lmax = sh_lmax_;
  p.dtype = dt;

  // kernel coverage: each (l, parity) at most once per string, one
  // multiplicity, l <= kMaxL, U <= 64
  const int U = p.in[0].mul;
  int lmax = sh_lmax_;
  bool repeated_l = false;
  for (const auto* v : {&p.in, &p.out}) {
    bool seen[64][2] = {};
    bool any[64] = {};
    for (const Segment& sg : *v) {
      if (sg.l > kMaxL)
        return fail(TPCONV_E_UNSUPPORTED, "l = " + std::to_string(sg.l) + " exceeds TPCONV_MAX_L");
      const int pi = sg.p > 0 ? 0 : 1;
      if (seen[sg.l][pi])
        return fail(TPCONV_E_UNSUPPORTED, "l = " + std::to_string(sg.l) + " with one parity appears twice in one irreps string");
      seen[sg.l][pi] = true;
      if (any[sg.l]) repeated_l = true;
      any[sg.l] = true;
      if (sg.mul != U) return fail(TPCONV_E_UNSUPPORTED, "all segments must share one multiplicity");
      lmax = std::max(lmax, sg.l);
    }
  }
  if (sh_lmax_ > kMaxL) return fail(TPCONV_E_UNSUPPORTED, "sh_lmax exceeds TPCONV_MAX_L");
  if (U > 64) return fail(TPCONV_E_UNSUPPORTED, "multiplicity above 64 is not supported by the kernels");
  p.mul = U;
  p.kernel_l = lmax;

  // dimensions and segment offsets
  p.dim_in = p.dim_out = 0;
  for (const Segment& sg : p.in) p.dim_in += sg.mul * (2 * sg.l + 1);
  for (const Segment& sg : p.out) p.dim_out += sg.mul * (2 * sg.l + 1);
  p.dim_sh = (sh_lmax_ + 1) * (sh_lmax_ + 1);

  // paths in lexicographic (s1, l2, s3) order
  p.paths.clear();
  int64_t woff = 0;
  for (int s1 = 0; s1 < static_cast<int>(p.in.size()); ++s1)
    for (int l2 = 0; l2 <= sh_lmax_; ++l2)
      for (int s3 = 0; s3 < static_cast<int>(p.out.size()); ++s3) {
        const Segment& a = p.in[s1];
        const Segment& c = p.out[s3];
        if (!cg::triangle(a.l, l2, c.l)) continue;
        const int py = (l2 % 2 == 0) ? 1 : -1;
        if (a.p * py != c.p) continue;
        p.paths.push_back(Path{s1, l2, s3, woff});
        woff += a.mul;
      }
  if (p.paths.empty()) return fail(TPCONV_E_NO_PATHS, "no admissible path between the given irreps");
  p.weight_numel = woff;

  // sparse real CG table: COO entries per path, |values| deduplicated
  p.entries.clear();
  p.path_ptr.assign(1, 0);
  p.values.clear();
  for (const Path& q : p.paths) {
    const int l1 = p.in[q.s1].l, l3 = p.out[q.s3].l;
    const cg::Table t = cg::build_table(l1, q.l2, l3);
    for (int k = 0; k < t.n; ++k) {
      const cg::Entry& e = t.e[k];
      int vi = -1;
      for (size_t v = 0; v < p.values.size(); ++v)
        if (std::fabs(p.values[v] - e.mag) <= 1e-14 * e.mag) {
          vi = static_cast<int>(v);
          break;
        }
      if (vi < 0) {
        vi = static_cast<int>(p.values.size());
        p.values.push_back(e.mag);
      }
      const uint32_t packed = static_cast<uint32_t>(e.m1) | (static_cast<uint32_t>(e.m2) << 4) |
                              (static_cast<uint32_t>(e.m3) << 8) | (static_cast<uint32_t>(e.neg) << 12) |
                              (static_cast<uint32_t>(vi) << 13);
      p.entries.push_back(packed);
    }
    p.path_ptr.push_back(static_cast<int32_t>(p.entries.size()));
  }

  // kernel arguments that depend only on the plan
  for (int l = 0; l <= kMaxL; ++l) p.in_off[l] = p.out_off[l] = -1;
  int off = 0;
  for (const Segment& sg : p.in) {
    p.in_off[sg.l] = off;
    off += sg.mul * (2 * sg.l + 1);
  }
  off = 0;
  for (const Segment& sg : p.out) {
    p.out_off[sg.l] = off;
    off += sg.mul * (2 * sg.l + 1);
  }
  for (int t = 0; t < kMaxTriples; ++t) p.woff[t] = -1;
  p.pmask_lo = p.pmask_hi = 0;
  for (const Path& q : p.paths) {
    const int t = triple_id(p.kernel_l, p.in[q.s1].l, q.l2, p.out[q.s3].l);
    if (t < 0) return fail(TPCONV_E_UNSUPPORTED, "internal: path outside the kernel's triple list");
    if (q.woff > INT32_MAX) return fail(TPCONV_E_UNSUPPORTED, "weight row wider than 2^31 columns");
    p.woff[t] = static_cast<int32_t>(q.woff);
    if (t < 64)
      p.pmask_lo |= 1ull << t;
    else
      p.pmask_hi |= 1ull << (t - 64);
  }
  if (!repeated_l) return TPCONV_OK;

  // both parities of some l: passes by segment type (t_in, t_out)
  auto type_of = [](const Segment& sg) { return sg.p * ((sg.l % 2 == 0) ? 1 : -1); };
  auto seg_offsets = [](const std::vector<Segment>& v, int type, int32_t (&off)[kMaxL + 1], int& n,
                        int (*tf)(const Segment&)) {
    for (int l = 0; l <= kMaxL; ++l) off[l] = -1;
    int o = 0;
    n = 0;
    for (const Segment& sg : v) {
      if (tf(sg) == type) {
        off[sg.l] = o;
        ++n;
      }
      o += sg.mul * (2 * sg.l + 1);
    }
  };
  int (*tf)(const Segment&) = type_of;
  for (int ti : {1, -1})
    for (int to : {1, -1}) {
      Pass ps;
      ps.t_in = ti;
      ps.t_out = to;
      seg_offsets(p.in, ti, ps.in_off, ps.n_in, tf);
      seg_offsets(p.out, to, ps.out_off, ps.n_out, tf);
      for (int t = 0; t < kMaxTriples; ++t) ps.woff[t] = -1;
      for (const Path& q : p.paths) {
        if (type_of(p.in[q.s1]) != ti || type_of(p.out[q.s3]) != to) continue;
        const int t = triple_id(p.kernel_l, p.in[q.s1].l, q.l2, p.out[q.s3].l);
        ps.woff[t] = static_cast<int32_t>(q.woff);
        if (t < 64)
          ps.pmask_lo |= 1ull << t;
        else
          ps.pmask_hi |= 1ull << (t - 64);
        ++ps.n_paths;
      }
      p.passes.push_back(ps);
    }
  return TPCONV_OK;
}

}  // namespace tpconv

using tpconv::fail;
using tpconv::Plan;

extern "C" tpconv_status tpconv_plan(const char* irreps_in, int sh_lmax, const char* irreps_out,
                                     tpconv_dtype dtype, tpconv_plan_t* out) {
  if (out == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL output handle");
  *out = nullptr;
  Plan* p = new (std::nothrow) Plan();
  if (p == nullptr) return fail(TPCONV_E_INVALID_ARG, "out of host memory");
  const tpconv_status st = Plan::build(irreps_in, sh_lmax, irreps_out, dtype, *p);
  if (st != TPCONV_OK) {
    delete p;
    return st;
  }
  *out = reinterpret_cast<tpconv_plan_t>(p);
  return TPCONV_OK;
}

extern "C" tpconv_status tpconv_plan_query(tpconv_plan_t h, tpconv_plan_info* info) {
  if (h == nullptr || info == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL plan or info");
  const Plan& p = *reinterpret_cast<const Plan*>(h);
  std::memset(info, 0, sizeof(*info));
  info->dim_in = p.dim_in;
  info->dim_out = p.dim_out;
  info->dim_sh = p.dim_sh;
  info->n_paths = static_cast<int64_t>(p.paths.size());
  info->weight_numel = p.weight_numel;
  info->cg_nnz = static_cast<int64_t>(p.entries.size());
  info->cg_nvalues = static_cast<int64_t>(p.values.size());
  info->mul = p.mul;
  info->kernel_lmax = p.kernel_l;
  info->dtype = p.dtype;
  return TPCONV_OK;
}

extern "C" tpconv_status tpconv_plan_paths(tpconv_plan_t h, int32_t* paths) {
  if (h == nullptr || paths == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL plan or buffer");
  const Plan& p = *reinterpret_cast<const Plan*>(h);
  for (size_t i = 0; i < p.paths.size(); ++i) {
    paths[4 * i + 0] = p.paths[i].s1;
    paths[4 * i + 1] = p.paths[i].l2;
    paths[4 * i + 2] = p.paths[i].s3;
    paths[4 * i + 3] = static_cast<int32_t>(p.paths[i].woff);
  }
  return TPCONV_OK;
}

extern "C" tpconv_status tpconv_plan_table(tpconv_plan_t h, uint32_t* entries, int32_t* path_ptr,
                                           double* values) {
  if (h == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL plan");
  const Plan& p = *reinterpret_cast<const Plan*>(h);
  if (entries) std::copy(p.entries.begin(), p.entries.end(), entries);
  if (path_ptr) std::copy(p.path_ptr.begin(), p.path_ptr.end(), path_ptr);
  if (values) std::copy(p.values.begin(), p.values.end(), values);
  return TPCONV_OK;
}

extern "C" void tpconv_plan_destroy(tpconv_plan_t h) { delete reinterpret_cast<Plan*>(h); }
