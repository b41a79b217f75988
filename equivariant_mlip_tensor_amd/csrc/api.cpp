// api.cpp -- tpconv_forward / tpconv_backward / tpconv_double_backward dispatch
// and error reporting.
#include <string>

#include "tpconv_internal.hpp"

namespace tpconv {

namespace {
thread_local std::string g_last_error;

using Launcher = hipError_t (*)(const KernelArgs&, hipStream_t);

enum class Kind { kFwd, kBwd, kDDF, kDDB };

Launcher pick(Kind k, int L, tpconv_dtype dt) {
  const bool f32 = dt == TPCONV_F32;
#define TPCONV_PICK(LL)                                                             \
  case LL:                                                                          \
    switch (k) {                                                                    \
      case Kind::kFwd: return f32 ? launch_fwd_l##LL##_f32 : launch_fwd_l##LL##_f64; \
      case Kind::kBwd: return f32 ? launch_bwd_l##LL##_f32 : launch_bwd_l##LL##_f64; \
      case Kind::kDDF: return f32 ? launch_ddf_l##LL##_f32 : launch_ddf_l##LL##_f64; \
      case Kind::kDDB: return f32 ? launch_ddb_l##LL##_f32 : launch_ddb_l##LL##_f64; \
    }                                                                               \
    return nullptr;
  switch (L) {
    TPCONV_PICK(0)
    TPCONV_PICK(1)
    TPCONV_PICK(2)
    TPCONV_PICK(3)
    TPCONV_PICK(4)
    default:
      return nullptr;
  }
#undef TPCONV_PICK
}

// The launch arguments of a plan, or of one of its passes (ps).
KernelArgs base_args(const Plan& p, int64_t n_rows, const Pass* ps = nullptr) {
  KernelArgs a{};
  a.n_rows = static_cast<int32_t>(n_rows);
  a.mul = p.mul;
  int lg = 0;
  while ((1 << lg) < p.mul) ++lg;
  a.lps_log2 = lg;
  a.nslots = 64 >> lg;
  a.d_in = static_cast<int32_t>(p.dim_in);
  a.d_out = static_cast<int32_t>(p.dim_out);
  a.d_sh = static_cast<int32_t>(p.dim_sh);
  a.wstride = p.weight_numel;
  a.pmask_lo = ps ? ps->pmask_lo : p.pmask_lo;
  a.pmask_hi = ps ? ps->pmask_hi : p.pmask_hi;
  for (int l = 0; l <= kMaxL; ++l) {
    a.in_off[l] = ps ? ps->in_off[l] : p.in_off[l];
    a.out_off[l] = ps ? ps->out_off[l] : p.out_off[l];
  }
  for (int t = 0; t < kMaxTriples; ++t) a.woff[t] = ps ? ps->woff[t] : p.woff[t];
  // first path into each output l in the forward's (l1, l2, l3) loop order,
  // and first path out of each input l in the backward's (l3, l1, l2) order
  const int L = p.kernel_l;
  auto on = [&](int t) { return t < 64 ? ((a.pmask_lo >> t) & 1ull) : ((a.pmask_hi >> (t - 64)) & 1ull); };
  auto set = [](uint64_t& lo, uint64_t& hi, int t) { (t < 64 ? lo : hi) |= 1ull << (t < 64 ? t : t - 64); };
  bool seen3[kMaxL + 1] = {}, seen1[kMaxL + 1] = {};
  for (int l1 = 0; l1 <= L; ++l1)
    for (int l2 = 0; l2 <= L; ++l2)
      for (int l3 = 0; l3 <= L; ++l3) {
        const int t = triple_id(L, l1, l2, l3);
        if (t < 0 || !on(t)) continue;
        if (!seen3[l3]) set(a.first3_lo, a.first3_hi, t);
        seen3[l3] = true;
        a.out_l_mask |= 1 << l3;
        a.in_l_mask |= 1 << l1;
      }
  for (int l3 = 0; l3 <= L; ++l3)
    for (int l1 = 0; l1 <= L; ++l1)
      for (int l2 = 0; l2 <= L; ++l2) {
        const int t = triple_id(L, l1, l2, l3);
        if (t < 0 || !on(t)) continue;
        if (!seen1[l1]) set(a.first1_lo, a.first1_hi, t);
        seen1[l1] = true;
      }
  // the compile-time ("full") kernels cover plans whose segments are l = 0..L
  // in order with natural parity on both sides and SH up to the same L
  bool full = p.sh_lmax == L && static_cast<int>(p.in.size()) == L + 1 && static_cast<int>(p.out.size()) == L + 1;
  for (int l = 0; full && l <= L; ++l) {
    const int par = (l % 2 == 0) ? 1 : -1;
    full = p.in[l].l == l && p.out[l].l == l && p.in[l].p == par && p.out[l].p == par;
  }
  a.full_plan = full && ps == nullptr ? 1 : 0;
  return a;
}

// The launches of a plan: the plan itself, or its passes ordered so that the
// first launch writing a group of segments overwrites them and the later
// ones add into them (KernelArgs::acc).
struct Launch {
  const Pass* pass;
  int acc;
};

// Launches over output segments (forward, double backward's grad_G): passes
// grouped by output type; a type no path reaches is written as zeros by one
// of its passes without paths.
std::vector<Launch> out_launches(const Plan& p) {
  if (p.passes.empty()) return {Launch{nullptr, 0}};
  std::vector<Launch> v;
  for (int to : {1, -1}) {
    bool first = true;
    const Pass* zero = nullptr;
    for (const Pass& ps : p.passes) {
      if (ps.t_out != to || ps.n_out == 0) continue;
      if (ps.n_paths == 0) {
        if (zero == nullptr) zero = &ps;
        continue;
      }
      v.push_back(Launch{&ps, first ? 0 : 1});
      first = false;
    }
    if (first && zero != nullptr) v.push_back(Launch{zero, 0});
  }
  return v;
}

// Launches over input segments (backward, double backward's second kernel):
// passes grouped by input type for grad_x (bit 0); every launch after the
// first adds into grad_Y (bit 1); each pass writes its own paths' grad_W.
std::vector<Launch> in_launches(const Plan& p) {
  if (p.passes.empty()) return {Launch{nullptr, 0}};
  std::vector<Launch> v;
  for (int ti : {1, -1}) {
    bool first = true;
    const Pass* zero = nullptr;
    for (const Pass& ps : p.passes) {
      if (ps.t_in != ti || ps.n_in == 0) continue;
      if (ps.n_paths == 0) {
        if (zero == nullptr) zero = &ps;
        continue;
      }
      v.push_back(Launch{&ps, first ? 0 : 1});
      first = false;
    }
    if (first && zero != nullptr) v.push_back(Launch{zero, 0});
  }
  for (size_t i = 1; i < v.size(); ++i) v[i].acc |= 2;
  return v;
}

}  // namespace

tpconv_status fail(tpconv_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

}  // namespace tpconv

using namespace tpconv;

extern "C" const char* tpconv_last_error(void) { return g_last_error.c_str(); }

extern "C" tpconv_status tpconv_forward(tpconv_plan_t hp, tpconv_graph_t hg, const void* x, const void* Y,
                                        const void* W, void* out, hipStream_t stream) {
  if (hp == nullptr || hg == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL plan or graph");
  const Plan& p = *reinterpret_cast<const Plan*>(hp);
  const Graph& g = *reinterpret_cast<const Graph*>(hg);
  if (g.n_nodes > 0 && (out == nullptr || x == nullptr)) return fail(TPCONV_E_INVALID_ARG, "NULL x or out");
  if (g.n_edges > 0 && (Y == nullptr || W == nullptr)) return fail(TPCONV_E_INVALID_ARG, "NULL Y or W");
  if (g.n_nodes == 0) return TPCONV_OK;
  Launcher f = pick(Kind::kFwd, p.kernel_l, p.dtype);
  if (f == nullptr) return fail(TPCONV_E_UNSUPPORTED, "no kernel for this l bound");
  for (const Launch& ln : out_launches(p)) {
    KernelArgs a = base_args(p, g.n_nodes, ln.pass);
    a.acc = ln.acc;
    a.row_ptr = g.dst_row;
    a.col = g.dst_col;
    a.eid = g.dst_eid;
    a.order = g.dst_order;
    a.x = x;
    a.Y = Y;
    a.W = W;
    a.out = out;
    const hipError_t he = f(a, stream);
    if (he != hipSuccess) return fail(TPCONV_E_HIP, std::string("forward launch: ") + hipGetErrorString(he));
  }
  return TPCONV_OK;
}

extern "C" tpconv_status tpconv_backward(tpconv_plan_t hp, tpconv_graph_t hg, const void* x, const void* Y,
                                         const void* W, const void* grad_out, void* grad_x, void* grad_Y,
                                         void* grad_W, hipStream_t stream) {
  if (hp == nullptr || hg == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL plan or graph");
  const Plan& p = *reinterpret_cast<const Plan*>(hp);
  const Graph& g = *reinterpret_cast<const Graph*>(hg);
  const bool want_edges = g.n_edges > 0 && (grad_Y != nullptr || grad_W != nullptr);
  if (grad_x == nullptr && !want_edges) return TPCONV_OK;
  if (g.n_nodes > 0 && (x == nullptr || grad_out == nullptr))
    return fail(TPCONV_E_INVALID_ARG, "NULL x or grad_out");
  if (g.n_edges > 0 && (Y == nullptr || W == nullptr)) return fail(TPCONV_E_INVALID_ARG, "NULL Y or W");
  if (g.n_nodes == 0) return TPCONV_OK;
  Launcher f = pick(Kind::kBwd, p.kernel_l, p.dtype);
  if (f == nullptr) return fail(TPCONV_E_UNSUPPORTED, "no kernel for this l bound");
  for (const Launch& ln : in_launches(p)) {
    KernelArgs a = base_args(p, g.n_nodes, ln.pass);
    a.acc = ln.acc;
    a.row_ptr = g.src_row;
    a.col = g.src_col;
    a.eid = g.src_eid;
    a.order = g.src_order;
    a.x = x;
    a.Y = Y;
    a.W = W;
    a.G = grad_out;
    a.out = grad_x;
    a.dY = grad_Y;
    a.dW = grad_W;
    const hipError_t he = f(a, stream);
    if (he != hipSuccess) return fail(TPCONV_E_HIP, std::string("backward launch: ") + hipGetErrorString(he));
  }
  return TPCONV_OK;
}

namespace {
// Plans the kernels that evaluate the harmonics themselves cover: every plan
// that runs as one launch per direction (not those holding both parities of
// some l, which run as passes adding into shared outputs).
tpconv_status vec_check(const Plan& p) {
  if (!p.passes.empty())
    return fail(TPCONV_E_UNSUPPORTED,
                "harmonics from edge vectors: plans holding both parities of one l run as several passes; use "
                "tpconv_sh, tpconv_forward, tpconv_backward and tpconv_sh_backward");
  return TPCONV_OK;
}
}  // namespace

extern "C" tpconv_status tpconv_forward_vec(tpconv_plan_t hp, tpconv_graph_t hg, const void* x, const void* vec,
                                            const void* W, void* out, hipStream_t stream) {
  if (hp == nullptr || hg == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL plan or graph");
  const Plan& p = *reinterpret_cast<const Plan*>(hp);
  const Graph& g = *reinterpret_cast<const Graph*>(hg);
  KernelArgs a = base_args(p, g.n_nodes);
  const tpconv_status st = vec_check(p);
  if (st != TPCONV_OK) return st;
  if (g.n_nodes > 0 && (out == nullptr || x == nullptr)) return fail(TPCONV_E_INVALID_ARG, "NULL x or out");
  if (g.n_edges > 0 && (vec == nullptr || W == nullptr)) return fail(TPCONV_E_INVALID_ARG, "NULL vec or W");
  if (g.n_nodes == 0) return TPCONV_OK;
  Launcher f = pick(Kind::kFwd, p.kernel_l, p.dtype);
  if (f == nullptr) return fail(TPCONV_E_UNSUPPORTED, "no kernel for this l bound");
  a.row_ptr = g.dst_row;
  a.col = g.dst_col;
  a.eid = g.dst_eid;
  a.order = g.dst_order;
  a.x = x;
  a.W = W;
  a.out = out;
  a.from_vec = 1;
  a.vec = vec;
  const hipError_t he = f(a, stream);
  if (he != hipSuccess) return fail(TPCONV_E_HIP, std::string("forward launch: ") + hipGetErrorString(he));
  return TPCONV_OK;
}

extern "C" tpconv_status tpconv_backward_vec(tpconv_plan_t hp, tpconv_graph_t hg, const void* x, const void* vec,
                                             const void* W, const void* grad_out, void* grad_x, void* grad_vec,
                                             void* grad_W, hipStream_t stream) {
  if (hp == nullptr || hg == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL plan or graph");
  const Plan& p = *reinterpret_cast<const Plan*>(hp);
  const Graph& g = *reinterpret_cast<const Graph*>(hg);
  KernelArgs a = base_args(p, g.n_nodes);
  const tpconv_status st = vec_check(p);
  if (st != TPCONV_OK) return st;
  const bool want_edges = g.n_edges > 0 && (grad_vec != nullptr || grad_W != nullptr);
  if (grad_x == nullptr && !want_edges) return TPCONV_OK;
  if (g.n_nodes > 0 && (x == nullptr || grad_out == nullptr))
    return fail(TPCONV_E_INVALID_ARG, "NULL x or grad_out");
  if (g.n_edges > 0 && (vec == nullptr || W == nullptr)) return fail(TPCONV_E_INVALID_ARG, "NULL vec or W");
  if (g.n_nodes == 0) return TPCONV_OK;
  Launcher f = pick(Kind::kBwd, p.kernel_l, p.dtype);
  if (f == nullptr) return fail(TPCONV_E_UNSUPPORTED, "no kernel for this l bound");
  a.row_ptr = g.src_row;
  a.col = g.src_col;
  a.eid = g.src_eid;
  a.order = g.src_order;
  a.x = x;
  a.W = W;
  a.G = grad_out;
  a.out = grad_x;
  a.dW = grad_W;
  a.from_vec = 1;
  a.vec = vec;
  a.gvec = g.n_edges > 0 ? grad_vec : nullptr;
  const hipError_t he = f(a, stream);
  if (he != hipSuccess) return fail(TPCONV_E_HIP, std::string("backward launch: ") + hipGetErrorString(he));
  return TPCONV_OK;
}

namespace {
using RadialLauncher = hipError_t (*)(bool, const KernelArgs&, const float*, const float*, float*, int, hipStream_t);

RadialLauncher pick_radial(int L) {
  switch (L) {
    case 0: return launch_radial_l0_f32;
    case 1: return launch_radial_l1_f32;
    case 2: return launch_radial_l2_f32;
    case 3: return launch_radial_l3_f32;
    case 4: return launch_radial_l4_f32;
    default: return nullptr;
  }
}

// Checks shared by the two radial entry points; lgH = log2(hidden) on success.
tpconv_status radial_check(const Plan& p, const KernelArgs& a, int hidden, const void* h, const void* M,
                           int64_t n_edges, int& lgH) {
  if (p.dtype != TPCONV_F32 || !a.full_plan || (p.mul != 16 && p.mul != 32 && p.mul != 64) || !p.passes.empty())
    return fail(TPCONV_E_UNSUPPORTED,
                "radial weights: fp32 plans with segments l = 0..L in order, natural parity, SH up to L and "
                "U in {16, 32, 64}");
  lgH = 0;
  while ((1 << lgH) < hidden) ++lgH;
  if (hidden < 16 || hidden > 128 || (1 << lgH) != hidden)
    return fail(TPCONV_E_UNSUPPORTED, "radial weights: hidden width must be 16, 32, 64 or 128");
  if (n_edges > 0 && (h == nullptr || M == nullptr)) return fail(TPCONV_E_INVALID_ARG, "NULL h or M");
  if (reinterpret_cast<uintptr_t>(M) % 16 != 0 || reinterpret_cast<uintptr_t>(h) % 16 != 0)
    return fail(TPCONV_E_INVALID_ARG, "radial weights: h and M must be 16-byte aligned");
  return TPCONV_OK;
}
}  // namespace

extern "C" tpconv_status tpconv_radial_forward(tpconv_plan_t hp, tpconv_graph_t hg, int hidden, const void* x,
                                               const void* Y, const void* h, const void* M, void* out,
                                               hipStream_t stream) {
  if (hp == nullptr || hg == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL plan or graph");
  const Plan& p = *reinterpret_cast<const Plan*>(hp);
  const Graph& g = *reinterpret_cast<const Graph*>(hg);
  KernelArgs a = base_args(p, g.n_nodes);
  int lgH = 0;
  const tpconv_status st = radial_check(p, a, hidden, h, M, g.n_edges, lgH);
  if (st != TPCONV_OK) return st;
  if (g.n_nodes > 0 && (out == nullptr || x == nullptr)) return fail(TPCONV_E_INVALID_ARG, "NULL x or out");
  if (g.n_edges > 0 && Y == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL Y");
  if (g.n_nodes == 0) return TPCONV_OK;
  RadialLauncher f = pick_radial(p.kernel_l);
  if (f == nullptr) return fail(TPCONV_E_UNSUPPORTED, "no kernel for this l bound");
  a.row_ptr = g.dst_row;
  a.col = g.dst_col;
  a.eid = g.dst_eid;
  a.order = g.dst_order;
  a.x = x;
  a.Y = Y;
  a.out = out;
  const hipError_t he = f(true, a, static_cast<const float*>(h), static_cast<const float*>(M), nullptr, lgH, stream);
  if (he == hipErrorInvalidValue) return fail(TPCONV_E_UNSUPPORTED, "radial weights: this plan's W tile exceeds LDS");
  if (he != hipSuccess) return fail(TPCONV_E_HIP, std::string("radial forward launch: ") + hipGetErrorString(he));
  return TPCONV_OK;
}

extern "C" tpconv_status tpconv_radial_backward(tpconv_plan_t hp, tpconv_graph_t hg, int hidden, const void* x,
                                                const void* Y, const void* h, const void* M, const void* grad_out,
                                                void* grad_x, void* grad_Y, void* grad_h, void* grad_W,
                                                hipStream_t stream) {
  if (hp == nullptr || hg == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL plan or graph");
  const Plan& p = *reinterpret_cast<const Plan*>(hp);
  const Graph& g = *reinterpret_cast<const Graph*>(hg);
  KernelArgs a = base_args(p, g.n_nodes);
  int lgH = 0;
  const tpconv_status st = radial_check(p, a, hidden, h, M, g.n_edges, lgH);
  if (st != TPCONV_OK) return st;
  const bool want_edges = g.n_edges > 0 && (grad_Y != nullptr || grad_h != nullptr || grad_W != nullptr);
  if (grad_x == nullptr && !want_edges) return TPCONV_OK;
  if (g.n_nodes > 0 && (x == nullptr || grad_out == nullptr)) return fail(TPCONV_E_INVALID_ARG, "NULL x or grad_out");
  if (g.n_edges > 0 && Y == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL Y");
  if (g.n_nodes == 0) return TPCONV_OK;
  RadialLauncher f = pick_radial(p.kernel_l);
  if (f == nullptr) return fail(TPCONV_E_UNSUPPORTED, "no kernel for this l bound");
  a.row_ptr = g.src_row;
  a.col = g.src_col;
  a.eid = g.src_eid;
  a.order = g.src_order;
  a.x = x;
  a.Y = Y;
  a.G = grad_out;
  a.out = grad_x;
  a.dY = grad_Y;
  a.dW = grad_W;
  const hipError_t he = f(false, a, static_cast<const float*>(h), static_cast<const float*>(M),
                          static_cast<float*>(grad_h), lgH, stream);
  if (he == hipErrorInvalidValue) return fail(TPCONV_E_UNSUPPORTED, "radial weights: this plan's W tile exceeds LDS");
  if (he != hipSuccess) return fail(TPCONV_E_HIP, std::string("radial backward launch: ") + hipGetErrorString(he));
  return TPCONV_OK;
}

extern "C" tpconv_status tpconv_double_backward(tpconv_plan_t hp, tpconv_graph_t hg, const void* x, const void* Y,
                                                const void* W, const void* grad_out, const void* ggx,
                                                const void* ggY, const void* ggW, void* grad_x, void* grad_Y,
                                                void* grad_W, void* grad_G, hipStream_t stream) {
  if (hp == nullptr || hg == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL plan or graph");
  const Plan& p = *reinterpret_cast<const Plan*>(hp);
  const Graph& g = *reinterpret_cast<const Graph*>(hg);
  const bool want_edges = g.n_edges > 0 && (grad_Y != nullptr || grad_W != nullptr);
  const bool want_src = grad_x != nullptr || want_edges;  // second kernel
  const bool want_dst = grad_G != nullptr;                 // first kernel
  if (!want_src && !want_dst) return TPCONV_OK;
  if (g.n_nodes > 0 && x == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL x");
  if (g.n_nodes > 0 && want_src && grad_out == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL grad_out");
  if (g.n_edges > 0 && (Y == nullptr || W == nullptr)) return fail(TPCONV_E_INVALID_ARG, "NULL Y or W");
  if (g.n_nodes == 0) return TPCONV_OK;
  Launcher ff = pick(Kind::kDDF, p.kernel_l, p.dtype);
  Launcher fb = pick(Kind::kDDB, p.kernel_l, p.dtype);
  if (ff == nullptr || fb == nullptr) return fail(TPCONV_E_UNSUPPORTED, "no kernel for this l bound");
  auto common = [&](const Launch& ln) {
    KernelArgs a = base_args(p, g.n_nodes, ln.pass);
    a.acc = ln.acc;
    a.x = x;
    a.Y = Y;
    a.W = W;
    a.xa = ggx;
    a.Yb = ggY;
    a.Wc = ggW;
    return a;
  };
  if (want_dst) {
    for (const Launch& ln : out_launches(p)) {
      KernelArgs f = common(ln);
      f.row_ptr = g.dst_row;
      f.col = g.dst_col;
      f.eid = g.dst_eid;
      f.order = g.dst_order;
      f.out = grad_G;
      const hipError_t he = ff(f, stream);
      if (he != hipSuccess) return fail(TPCONV_E_HIP, std::string("double backward launch: ") + hipGetErrorString(he));
    }
  }
  if (want_src) {
    for (const Launch& ln : in_launches(p)) {
      KernelArgs b = common(ln);
      b.row_ptr = g.src_row;
      b.col = g.src_col;
      b.eid = g.src_eid;
      b.order = g.src_order;
      b.G = grad_out;
      b.out = grad_x;
      b.dY = grad_Y;
      b.dW = grad_W;
      const hipError_t he = fb(b, stream);
      if (he != hipSuccess) return fail(TPCONV_E_HIP, std::string("double backward launch: ") + hipGetErrorString(he));
    }
  }
  return TPCONV_OK;
}

extern "C" tpconv_status tpconv_sh(tpconv_plan_t hp, int64_t n_edges, const void* vec, void* Y, hipStream_t stream) {
  if (hp == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL plan");
  if (n_edges < 0) return fail(TPCONV_E_INVALID_ARG, "n_edges < 0");
  if (n_edges > 0 && (vec == nullptr || Y == nullptr)) return fail(TPCONV_E_INVALID_ARG, "NULL vec or Y");
  const Plan& p = *reinterpret_cast<const Plan*>(hp);
  const hipError_t he = launch_sh(p.sh_lmax, p.dtype == TPCONV_F64, n_edges, vec, Y, stream);
  if (he != hipSuccess) return fail(TPCONV_E_HIP, std::string("sh launch: ") + hipGetErrorString(he));
  return TPCONV_OK;
}

extern "C" tpconv_status tpconv_sh_backward(tpconv_plan_t hp, int64_t n_edges, const void* vec, const void* grad_Y,
                                            void* grad_vec, hipStream_t stream) {
  if (hp == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL plan");
  if (n_edges < 0) return fail(TPCONV_E_INVALID_ARG, "n_edges < 0");
  if (n_edges > 0 && (vec == nullptr || grad_Y == nullptr || grad_vec == nullptr))
    return fail(TPCONV_E_INVALID_ARG, "NULL vec, grad_Y or grad_vec");
  const Plan& p = *reinterpret_cast<const Plan*>(hp);
  const hipError_t he = launch_sh_backward(p.sh_lmax, p.dtype == TPCONV_F64, n_edges, vec, grad_Y, grad_vec, stream);
  if (he != hipSuccess) return fail(TPCONV_E_HIP, std::string("sh backward launch: ") + hipGetErrorString(he));
  return TPCONV_OK;
}

extern "C" tpconv_status tpconv_positions_backward(tpconv_plan_t hp, tpconv_graph_t hg, const void* grad_vec,
                                                   void* grad_pos, hipStream_t stream) {
  if (hp == nullptr || hg == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL plan or graph");
  const Plan& p = *reinterpret_cast<const Plan*>(hp);
  const Graph& g = *reinterpret_cast<const Graph*>(hg);
  if (g.n_nodes > 0 && grad_pos == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL grad_pos");
  if (g.n_edges > 0 && grad_vec == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL grad_vec");
  const hipError_t he = launch_pos_backward(p.dtype == TPCONV_F64, g.n_nodes, g.src_row, g.src_eid, g.dst_row,
                                            g.dst_eid, grad_vec, grad_pos, stream);
  if (he != hipSuccess) return fail(TPCONV_E_HIP, std::string("positions backward launch: ") + hipGetErrorString(he));
  return TPCONV_OK;
}

namespace {
bool so2_supported(int L, int C) { return L >= 1 && L <= 3 && (C == 16 || C == 32); }
}  // namespace

extern "C" int64_t tpconv_so2_weight_numel(int lmax, int channels) {
  return so2_supported(lmax, channels) ? so2_weight_numel(lmax, channels) : 0;
}

extern "C" tpconv_status tpconv_so2_rotations(int lmax, tpconv_dtype dtype, int64_t n_edges, const void* vec,
                                              void* D, hipStream_t stream) {
  if (n_edges < 0) return fail(TPCONV_E_INVALID_ARG, "n_edges < 0");
  if (lmax < 0 || lmax > 4) return fail(TPCONV_E_UNSUPPORTED, "SO(2) rotations: lmax must be 0..4");
  if (dtype != TPCONV_F32 && dtype != TPCONV_F64) return fail(TPCONV_E_INVALID_ARG, "unknown dtype");
  if (n_edges > 0 && (vec == nullptr || D == nullptr)) return fail(TPCONV_E_INVALID_ARG, "NULL vec or D");
  const hipError_t he = launch_so2_wigner(lmax, dtype == TPCONV_F64, n_edges, vec, D, stream);
  if (he != hipSuccess) return fail(TPCONV_E_HIP, std::string("SO(2) rotations launch: ") + hipGetErrorString(he));
  return TPCONV_OK;
}

extern "C" tpconv_status tpconv_so2_forward(tpconv_graph_t hg, int lmax, int channels, tpconv_dtype dtype,
                                            const void* x, const void* D, const void* weights, void* out,
                                            hipStream_t stream) {
  if (hg == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL graph");
  if (!so2_supported(lmax, channels) || dtype != TPCONV_F32)
    return fail(TPCONV_E_UNSUPPORTED, "SO(2) convolution: lmax 1..3, channels 16 or 32, fp32");
  const Graph& g = *reinterpret_cast<const Graph*>(hg);
  if (g.n_nodes == 0) return TPCONV_OK;
  if (out == nullptr || weights == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL out or weights");
  if (reinterpret_cast<uintptr_t>(weights) % 16 != 0)
    return fail(TPCONV_E_INVALID_ARG, "SO(2) weights must be 16-byte aligned");
  if (g.n_edges > 0 && (x == nullptr || D == nullptr)) return fail(TPCONV_E_INVALID_ARG, "NULL x or D");
  const hipError_t he = launch_so2_conv(lmax, channels, false, false, (int)g.n_nodes, g.dst_row, g.dst_col, g.dst_eid,
                                        g.dst_order, static_cast<const float*>(x), static_cast<const float*>(D),
                                        static_cast<const float*>(weights), static_cast<float*>(out), nullptr, nullptr,
                                        stream);
  if (he != hipSuccess) return fail(TPCONV_E_HIP, std::string("SO(2) forward launch: ") + hipGetErrorString(he));
  return TPCONV_OK;
}

extern "C" size_t tpconv_so2_workspace_bytes(int lmax, int channels, int64_t n_edges) {
  if (!so2_supported(lmax, channels) || n_edges < 0) return 0;
  return (size_t)(so2_wgrad_blocks(n_edges) + 1) * (size_t)so2_weight_numel(lmax, channels) * sizeof(float);
}

extern "C" tpconv_status tpconv_so2_backward(tpconv_graph_t hg, int lmax, int channels, tpconv_dtype dtype,
                                             const void* x, const void* D, const void* weights, const void* grad_out,
                                             void* grad_x, void* grad_weights, void* workspace,
                                             size_t workspace_bytes, hipStream_t stream) {
  if (hg == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL graph");
  if (!so2_supported(lmax, channels) || dtype != TPCONV_F32)
    return fail(TPCONV_E_UNSUPPORTED, "SO(2) convolution: lmax 1..3, channels 16 or 32, fp32");
  const Graph& g = *reinterpret_cast<const Graph*>(hg);
  if (grad_x == nullptr && grad_weights == nullptr) return TPCONV_OK;
  const size_t need = tpconv_so2_workspace_bytes(lmax, channels, g.n_edges);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(TPCONV_E_WORKSPACE, "SO(2) backward: workspace smaller than tpconv_so2_workspace_bytes()");
  float* const ws_maps = static_cast<float*>(workspace);  // the transposed maps, weight_numel floats
  float* const ws_part = ws_maps + so2_weight_numel(lmax, channels);
  if (g.n_nodes > 0 && grad_out == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL grad_out");
  if (grad_x != nullptr && weights == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL weights");
  if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
    return fail(TPCONV_E_INVALID_ARG, "SO(2) workspace must be 16-byte aligned");
  if (g.n_edges > 0 && (x == nullptr || D == nullptr)) return fail(TPCONV_E_INVALID_ARG, "NULL x or D");
  if (grad_x != nullptr && g.n_nodes > 0) {
    const hipError_t he = launch_so2_conv(lmax, channels, true, false, (int)g.n_nodes, g.src_row, g.src_col, g.src_eid,
                                          g.src_order, static_cast<const float*>(grad_out),
                                          static_cast<const float*>(D), static_cast<const float*>(weights),
                                          static_cast<float*>(grad_x), ws_maps, nullptr, stream);
    if (he != hipSuccess) return fail(TPCONV_E_HIP, std::string("SO(2) backward launch: ") + hipGetErrorString(he));
  }
  if (grad_weights != nullptr) {
    const hipError_t he = launch_so2_wgrad(lmax, channels, (int)g.n_nodes, g.n_edges, g.dst_row, g.dst_col,
                                           g.dst_eid, static_cast<const float*>(x), static_cast<const float*>(grad_out),
                                           static_cast<const float*>(D), ws_part,
                                           static_cast<float*>(grad_weights), 0, stream);
    if (he != hipSuccess)
      return fail(TPCONV_E_HIP, std::string("SO(2) weight-gradient launch: ") + hipGetErrorString(he));
  }
  return TPCONV_OK;
}

extern "C" tpconv_status tpconv_so2_backward_noalloc(tpconv_graph_t hg, int lmax, int channels, tpconv_dtype dtype,
                                                     const void* x, const void* D, const void* weights,
                                                     const void* grad_out, void* grad_x, void* grad_weights,
                                                     hipStream_t stream) {
  if (hg == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL graph");
  if (!so2_supported(lmax, channels) || dtype != TPCONV_F32)
    return fail(TPCONV_E_UNSUPPORTED, "SO(2) convolution: lmax 1..3, channels 16 or 32, fp32");
  const Graph& g = *reinterpret_cast<const Graph*>(hg);
  if (grad_x == nullptr && grad_weights == nullptr) return TPCONV_OK;
  if (g.n_nodes > 0 && grad_out == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL grad_out");
  if (grad_x != nullptr && weights == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL weights");
  if (g.n_edges > 0 && (x == nullptr || D == nullptr)) return fail(TPCONV_E_INVALID_ARG, "NULL x or D");
  // the library's device scratch: the transposed maps, then as many blocks'
  // partial map gradients as fit (fewer blocks than the workspace entry
  // point uses when the scratch is the limit; each block then takes more edges)
  float* ws = nullptr;
  int64_t ws_floats = 0;
  const hipError_t se = so2_scratch(&ws, &ws_floats);
  if (se != hipSuccess) return fail(TPCONV_E_HIP, std::string("SO(2) scratch lookup: ") + hipGetErrorString(se));
  const int64_t nw = so2_weight_numel(lmax, channels);
  const int64_t max_blocks = ws_floats / nw - 1;
  if (max_blocks < 1)
    return fail(TPCONV_E_WORKSPACE, "SO(2) backward (no allocation): the maps (" + std::to_string(nw) +
                                        " floats) exceed the library scratch (" + std::to_string(ws_floats) +
                                        " floats)");
  if (grad_x != nullptr && g.n_nodes > 0) {
    const hipError_t he = launch_so2_conv(lmax, channels, true, false, (int)g.n_nodes, g.src_row, g.src_col, g.src_eid,
                                          g.src_order, static_cast<const float*>(grad_out),
                                          static_cast<const float*>(D), static_cast<const float*>(weights),
                                          static_cast<float*>(grad_x), ws, nullptr, stream);
    if (he != hipSuccess) return fail(TPCONV_E_HIP, std::string("SO(2) backward launch: ") + hipGetErrorString(he));
  }
  if (grad_weights != nullptr) {
    const hipError_t he = launch_so2_wgrad(lmax, channels, (int)g.n_nodes, g.n_edges, g.dst_row, g.dst_col,
                                           g.dst_eid, static_cast<const float*>(x), static_cast<const float*>(grad_out),
                                           static_cast<const float*>(D), ws + nw,
                                           static_cast<float*>(grad_weights), (int)max_blocks, stream);
    if (he != hipSuccess)
      return fail(TPCONV_E_HIP, std::string("SO(2) weight-gradient launch: ") + hipGetErrorString(he));
  }
  return TPCONV_OK;
}

extern "C" tpconv_status tpconv_so2_double_backward(tpconv_graph_t hg, int lmax, int channels, tpconv_dtype dtype,
                                                    const void* x, const void* D, const void* weights,
                                                    const void* grad_out, const void* ggx, const void* ggw,
                                                    void* grad_x, void* grad_weights, void* grad_G, void* workspace,
                                                    size_t workspace_bytes, hipStream_t stream) {
  if (hg == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL graph");
  if (!so2_supported(lmax, channels) || dtype != TPCONV_F32)
    return fail(TPCONV_E_UNSUPPORTED, "SO(2) convolution: lmax 1..3, channels 16 or 32, fp32");
  const Graph& g = *reinterpret_cast<const Graph*>(hg);
  if (grad_x == nullptr && grad_weights == nullptr && grad_G == nullptr) return TPCONV_OK;
  if (grad_x != nullptr || grad_weights != nullptr) {
    const size_t need = tpconv_so2_workspace_bytes(lmax, channels, g.n_edges);
    if (workspace == nullptr || workspace_bytes < need)
      return fail(TPCONV_E_WORKSPACE, "SO(2) double backward: workspace smaller than tpconv_so2_workspace_bytes()");
    if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
      return fail(TPCONV_E_INVALID_ARG, "SO(2) workspace must be 16-byte aligned");
  }
  const bool need_x = g.n_nodes > 0 && (ggw != nullptr || ggx != nullptr);
  if (need_x && (x == nullptr || D == nullptr)) return fail(TPCONV_E_INVALID_ARG, "NULL x or D");
  if (g.n_nodes > 0 && (grad_x != nullptr || grad_weights != nullptr) && grad_out == nullptr)
    return fail(TPCONV_E_INVALID_ARG, "NULL grad_out");
  if (grad_G != nullptr && ggx != nullptr && weights == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL weights");
  if ((weights != nullptr && reinterpret_cast<uintptr_t>(weights) % 16 != 0) ||
      (ggw != nullptr && reinterpret_cast<uintptr_t>(ggw) % 16 != 0))
    return fail(TPCONV_E_INVALID_ARG, "SO(2) weights and ggw must be 16-byte aligned");
  const int64_t nw = so2_weight_numel(lmax, channels);
  const int64_t nd = g.n_nodes * (int64_t)channels * (lmax + 1) * (lmax + 1);
  float* const ws_maps = static_cast<float*>(workspace);
  float* const ws_part = ws_maps == nullptr ? nullptr : ws_maps + nw;
  const float* fx = static_cast<const float*>(x);
  const float* fD = static_cast<const float*>(D);
  const float* fG = static_cast<const float*>(grad_out);
  auto check = [](hipError_t he, const char* what) -> tpconv_status {
    if (he != hipSuccess) return fail(TPCONV_E_HIP, std::string(what) + hipGetErrorString(he));
    return TPCONV_OK;
  };
  tpconv_status st = TPCONV_OK;
  // grad_G = f(ggx; w) + f(x; ggw)
  if (grad_G != nullptr) {
    float* out = static_cast<float*>(grad_G);
    if (ggx != nullptr)
      st = check(launch_so2_conv(lmax, channels, false, false, (int)g.n_nodes, g.dst_row, g.dst_col, g.dst_eid,
                                 g.dst_order, static_cast<const float*>(ggx), fD, static_cast<const float*>(weights),
                                 out, nullptr, nullptr, stream),
                 "SO(2) double backward launch: ");
    if (st == TPCONV_OK && ggw != nullptr)
      st = check(launch_so2_conv(lmax, channels, false, ggx != nullptr, (int)g.n_nodes, g.dst_row, g.dst_col,
                                 g.dst_eid, g.dst_order, fx, fD, static_cast<const float*>(ggw), out, nullptr,
                                 nullptr, stream),
                 "SO(2) double backward launch: ");
    if (st == TPCONV_OK && ggx == nullptr && ggw == nullptr)
      st = check(launch_so2_fill_zero(nd, out, stream), "SO(2) double backward fill: ");
    if (st != TPCONV_OK) return st;
  }
  // grad_x = f(.; ggw)^T grad_out
  if (grad_x != nullptr) {
    float* out = static_cast<float*>(grad_x);
    st = ggw != nullptr
             ? check(launch_so2_conv(lmax, channels, true, false, (int)g.n_nodes, g.src_row, g.src_col, g.src_eid,
                                     g.src_order, fG, fD, static_cast<const float*>(ggw), out, ws_maps, nullptr,
                                     stream),
                     "SO(2) double backward launch: ")
             : check(launch_so2_fill_zero(nd, out, stream), "SO(2) double backward fill: ");
    if (st != TPCONV_OK) return st;
  }
  // grad_w = map gradient of (ggx, grad_out)
  if (grad_weights != nullptr) {
    float* out = static_cast<float*>(grad_weights);
    st = ggx != nullptr
             ? check(launch_so2_wgrad(lmax, channels, (int)g.n_nodes, g.n_edges, g.dst_row, g.dst_col, g.dst_eid,
                                      static_cast<const float*>(ggx), fG, fD, ws_part, out, 0, stream),
                     "SO(2) double backward launch: ")
             : check(launch_so2_fill_zero(nw, out, stream), "SO(2) double backward fill: ");
  }
  return st;
}

extern "C" tpconv_status tpconv_so2_frames_backward(tpconv_graph_t hg, int lmax, int channels, tpconv_dtype dtype,
                                                    const void* x, const void* D, const void* weights,
                                                    const void* grad_out, void* grad_D, void* workspace,
                                                    size_t workspace_bytes, hipStream_t stream) {
  if (hg == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL graph");
  if (!so2_supported(lmax, channels) || dtype != TPCONV_F32)
    return fail(TPCONV_E_UNSUPPORTED, "SO(2) convolution: lmax 1..3, channels 16 or 32, fp32");
  const Graph& g = *reinterpret_cast<const Graph*>(hg);
  if (grad_D == nullptr || g.n_edges == 0) return TPCONV_OK;
  const size_t need = tpconv_so2_workspace_bytes(lmax, channels, g.n_edges);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(TPCONV_E_WORKSPACE, "SO(2) frames backward: workspace smaller than tpconv_so2_workspace_bytes()");
  if (x == nullptr || D == nullptr || weights == nullptr || grad_out == nullptr)
    return fail(TPCONV_E_INVALID_ARG, "NULL x, D, weights or grad_out");
  if (reinterpret_cast<uintptr_t>(weights) % 16 != 0 || reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
    return fail(TPCONV_E_INVALID_ARG, "SO(2) weights and workspace must be 16-byte aligned");
  const float* fx = static_cast<const float*>(x);
  const float* fG = static_cast<const float*>(grad_out);
  const float* fD = static_cast<const float*>(D);
  const float* fW = static_cast<const float*>(weights);
  float* out = static_cast<float*>(grad_D);
  // the y~ G^T term over the destination rows (overwrites), then the dx~ x^T term over the source rows (adds)
  hipError_t he = launch_so2_conv(lmax, channels, false, false, (int)g.n_nodes, g.dst_row, g.dst_col, g.dst_eid,
                                  g.dst_order, fx, fD, fW, out, nullptr, fG, stream);
  if (he == hipSuccess)
    he = launch_so2_conv(lmax, channels, true, true, (int)g.n_nodes, g.src_row, g.src_col, g.src_eid, g.src_order,
                         fG, fD, fW, out, static_cast<float*>(workspace), fx, stream);
  if (he != hipSuccess) return fail(TPCONV_E_HIP, std::string("SO(2) frames backward launch: ") + hipGetErrorString(he));
  return TPCONV_OK;
}

extern "C" tpconv_status tpconv_so2_rotations_jvp(int lmax, tpconv_dtype dtype, int64_t n_edges, const void* vec,
                                                  const void* dvec, void* dD, hipStream_t stream) {
  if (n_edges < 0) return fail(TPCONV_E_INVALID_ARG, "n_edges < 0");
  if (lmax < 0 || lmax > 4) return fail(TPCONV_E_UNSUPPORTED, "SO(2) rotations: lmax must be 0..4");
  if (dtype != TPCONV_F32 && dtype != TPCONV_F64) return fail(TPCONV_E_INVALID_ARG, "unknown dtype");
  if (n_edges > 0 && (vec == nullptr || dvec == nullptr || dD == nullptr))
    return fail(TPCONV_E_INVALID_ARG, "NULL vec, dvec or dD");
  const hipError_t he = launch_so2_wigner_jvp(lmax, dtype == TPCONV_F64, n_edges, vec, dvec, dD, stream);
  if (he != hipSuccess) return fail(TPCONV_E_HIP, std::string("SO(2) rotations jvp launch: ") + hipGetErrorString(he));
  return TPCONV_OK;
}

namespace {
// Workspace of tpconv_so2_frames_double_backward: dD with the frames' roll
// projected out, the two terms of the map gradient, then the backward's
// workspace (transposed maps, block partials).
struct FddLayout {
  size_t ddp, wa, wb, so2, total;
};

FddLayout fdd_layout(int lmax, int C, int64_t n_edges) {
  FddLayout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = (o + bytes + 255) / 256 * 256;
    return at;
  };
  const int64_t nw = so2_weight_numel(lmax, C);
  const int64_t nd = int64_t(lmax + 1) * (2 * lmax + 1) * (2 * lmax + 3) / 3;
  L.ddp = take(sizeof(float) * nd * n_edges);
  L.wa = take(sizeof(float) * nw);
  L.wb = take(sizeof(float) * nw);
  L.so2 = take(tpconv_so2_workspace_bytes(lmax, C, n_edges));
  L.total = o;
  return L;
}
}  // namespace

extern "C" size_t tpconv_so2_frames_double_backward_workspace_bytes(int lmax, int channels, int64_t n_nodes,
                                                                    int64_t n_edges) {
  if (!so2_supported(lmax, channels) || n_nodes < 0 || n_edges < 0) return 0;
  return fdd_layout(lmax, channels, n_edges).total;
}

extern "C" tpconv_status tpconv_so2_frames_double_backward(tpconv_graph_t hg, int lmax, int channels,
                                                           tpconv_dtype dtype, const void* x, const void* D,
                                                           const void* weights, const void* grad_out, const void* dD,
                                                           void* grad_x, void* grad_weights, void* grad_G,
                                                           void* workspace, size_t workspace_bytes,
                                                           hipStream_t stream) {
  if (hg == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL graph");
  if (!so2_supported(lmax, channels) || dtype != TPCONV_F32)
    return fail(TPCONV_E_UNSUPPORTED, "SO(2) convolution: lmax 1..3, channels 16 or 32, fp32");
  const Graph& g = *reinterpret_cast<const Graph*>(hg);
  if (grad_x == nullptr && grad_weights == nullptr && grad_G == nullptr) return TPCONV_OK;
  const FddLayout L = fdd_layout(lmax, channels, g.n_edges);
  if (workspace == nullptr || workspace_bytes < L.total)
    return fail(TPCONV_E_WORKSPACE,
                "SO(2) frames double backward: workspace smaller than tpconv_so2_frames_double_backward_workspace_bytes()");
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(TPCONV_E_WORKSPACE, "SO(2) frames double backward: workspace must be 256-byte aligned");
  if (g.n_nodes > 0 && (x == nullptr || grad_out == nullptr)) return fail(TPCONV_E_INVALID_ARG, "NULL x or grad_out");
  if (weights == nullptr) return fail(TPCONV_E_INVALID_ARG, "NULL weights");
  if (reinterpret_cast<uintptr_t>(weights) % 16 != 0)
    return fail(TPCONV_E_INVALID_ARG, "SO(2) weights must be 16-byte aligned");
  if (g.n_edges > 0 && (D == nullptr || dD == nullptr)) return fail(TPCONV_E_INVALID_ARG, "NULL D or dD");
  char* base = static_cast<char*>(workspace);
  auto F = [&](size_t off) { return reinterpret_cast<float*>(base + off); };
  const int64_t nw = so2_weight_numel(lmax, channels);
  const float* fx = static_cast<const float*>(x);
  const float* fG = static_cast<const float*>(grad_out);
  const float* fW = static_cast<const float*>(weights);
  const float* fD = static_cast<const float*>(D);
  float* ws_maps = F(L.so2);
  float* ws_part = ws_maps + nw;
  const int n = (int)g.n_nodes;
  // the same second derivatives from dD less its roll component (exact; the
  // terms of a frames' derivative then no longer cancel)
  const float* fdD = F(L.ddp);
  hipError_t he = launch_so2_unroll(lmax, g.n_edges, fD, static_cast<const float*>(dD), F(L.ddp), stream);
  // grad_G over the destination rows: dD^T SO2(D x), then (adding) D^T SO2(dD x)
  if (he == hipSuccess && grad_G != nullptr && n > 0) {
    float* out = static_cast<float*>(grad_G);
    he = launch_so2_conv(lmax, channels, false, false, n, g.dst_row, g.dst_col, g.dst_eid, g.dst_order, fx, fD, fW,
                         out, nullptr, nullptr, stream, fdD);
    if (he == hipSuccess)
      he = launch_so2_conv(lmax, channels, false, true, n, g.dst_row, g.dst_col, g.dst_eid, g.dst_order, fx, fdD, fW,
                           out, nullptr, nullptr, stream, fD);
  }
  // grad_x over the source rows: D^T SO2^T(dD g), then (adding) dD^T SO2^T(D g)
  if (he == hipSuccess && grad_x != nullptr && n > 0) {
    float* out = static_cast<float*>(grad_x);
    he = launch_so2_conv(lmax, channels, true, false, n, g.src_row, g.src_col, g.src_eid, g.src_order, fG, fdD, fW,
                         out, ws_maps, nullptr, stream, fD);
    if (he == hipSuccess)
      he = launch_so2_conv(lmax, channels, true, true, n, g.src_row, g.src_col, g.src_eid, g.src_order, fG, fD, fW,
                           out, ws_maps, nullptr, stream, fdD);
  }
  // grad_weights: the map gradients of (dD g, D x) and (D g, dD x)
  if (he == hipSuccess && grad_weights != nullptr) {
    he = launch_so2_wgrad(lmax, channels, n, g.n_edges, g.dst_row, g.dst_col, g.dst_eid, fx, fG, fD, ws_part, F(L.wa),
                          0, stream, fdD);
    if (he == hipSuccess)
      he = launch_so2_wgrad(lmax, channels, n, g.n_edges, g.dst_row, g.dst_col, g.dst_eid, fx, fG, fdD, ws_part,
                            F(L.wb), 0, stream, fD);
    if (he == hipSuccess) he = launch_so2_add(nw, F(L.wa), F(L.wb), static_cast<float*>(grad_weights), stream);
  }
  if (he != hipSuccess)
    return fail(TPCONV_E_HIP, std::string("SO(2) frames double backward launch: ") + hipGetErrorString(he));
  return TPCONV_OK;
}

extern "C" tpconv_status tpconv_so2_rotations_backward(int lmax, tpconv_dtype dtype, int64_t n_edges, const void* vec,
                                                       const void* grad_D, void* grad_vec, hipStream_t stream) {
  if (n_edges < 0) return fail(TPCONV_E_INVALID_ARG, "n_edges < 0");
  if (lmax < 0 || lmax > 4) return fail(TPCONV_E_UNSUPPORTED, "SO(2) rotations: lmax must be 0..4");
  if (dtype != TPCONV_F32 && dtype != TPCONV_F64) return fail(TPCONV_E_INVALID_ARG, "unknown dtype");
  if (n_edges > 0 && (vec == nullptr || grad_D == nullptr || grad_vec == nullptr))
    return fail(TPCONV_E_INVALID_ARG, "NULL vec, grad_D or grad_vec");
  const hipError_t he = launch_so2_wigner_backward(lmax, dtype == TPCONV_F64, n_edges, vec, grad_D, grad_vec, stream);
  if (he != hipSuccess)
    return fail(TPCONV_E_HIP, std::string("SO(2) rotations backward launch: ") + hipGetErrorString(he));
  return TPCONV_OK;
}

