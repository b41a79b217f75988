"""GPU parity of tpconv_double_backward (through the C ABI) against the fp64 oracle.

Same metric and bounds as the forward/backward parity tests, per output
tensor (grad_x, grad_Y, grad_W, grad_G): max |T_gpu - T_ref| / rms(T_ref)
<= 1e-5 (fp32) or 1e-11 (fp64).  Full-size workloads compare sampled
destination rows (grad_G: every in-edge of the row), source rows (grad_x:
every out-edge) and edges (grad_Y, grad_W), each of which the oracle computes
exactly from the edges that feed it.
"""

import sys
import time
import zlib

import numpy as np
import pytest

import workloads
from oracle import TPProblem, tp_double_backward

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f64": 1e-11}
NAMES = ("grad_x", "grad_Y", "grad_W", "grad_G")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def tp():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
    from equivariant_mlip_tensor_amd import tpconv
    return tpconv


def rel_err(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape
    if ref.size == 0:
        return 0.0
    rms = np.sqrt(np.mean(ref ** 2))
    if rms == 0.0:
        return float(np.max(np.abs(gpu)))
    return float(np.max(np.abs(gpu - ref)) / rms)


def run_dd(tp, spec, n_nodes, src, dst, x, Y, W, G, a, b, c, need=(True, True, True, True)):
    import torch
    irr_in, lsh, irr_out, dt = spec
    plan = tp.tpconv_plan(irr_in, lsh, irr_out, dt)
    dev = torch.device("cuda:0")
    t = lambda v: None if v is None else torch.from_numpy(np.ascontiguousarray(v)).to(dev)  # noqa: E731
    g = tp.tpconv_graph_create(n_nodes, t(np.asarray(src, np.int32)), t(np.asarray(dst, np.int32)))
    outs = tp.tpconv_double_backward(plan, g, t(x), t(Y), t(W), t(G), t(a), t(b), t(c), need=need)
    torch.cuda.synchronize()
    return [None if o is None else o.cpu().numpy() for o in outs]


def random_case(spec, n_nodes, src, dst, seed):
    irr_in, lsh, irr_out, dt = spec
    prob = TPProblem.build(irr_in, lsh, irr_out)
    rng = np.random.default_rng(seed)
    npdt = np.float32 if dt == "f32" else np.float64
    E = len(src)
    x = rng.standard_normal((n_nodes, prob.dim_in)).astype(npdt)
    Y = (workloads.real_sh(lsh, rng.standard_normal((E, 3))).astype(npdt) if E
         else np.zeros((0, (lsh + 1) ** 2), npdt))
    W = (rng.standard_normal((E, prob.weight_numel)) / np.sqrt(len(prob.paths))).astype(npdt)
    G = rng.standard_normal((n_nodes, prob.dim_out)).astype(npdt)
    a = rng.standard_normal((n_nodes, prob.dim_in)).astype(npdt)
    b = rng.standard_normal((E, prob.dim_sh)).astype(npdt)
    c = rng.standard_normal((E, prob.weight_numel)).astype(npdt)
    return prob, x, Y, W, G, a, b, c


def check(got, ref, dt, label):
    errs = {k: rel_err(u, v) for k, u, v in zip(NAMES, got, ref)}
    log(f"[dd] {label} errors {errs}")
    for k, v in errs.items():
        assert v <= TOL[dt], (label, k, v)


def check_full(tp, spec, n_nodes, src, dst, seed=0, label="", drop=()):
    prob, x, Y, W, G, a, b, c = random_case(spec, n_nodes, src, dst, seed)
    cot = [None if k in drop else v for k, v in zip("abc", (a, b, c))]
    log(f"[dd] {label} spec={spec} N={n_nodes} E={len(src)} dropped={drop}")
    got = run_dd(tp, spec, n_nodes, src, dst, x, Y, W, G, *cot)
    ref = tp_double_backward(prob, x, Y, W, G, *cot, src, dst, n_nodes)
    check(got, ref, spec[3], label)
    return got


# ------------------------------------------------------------------ workloads
def workload_inputs(name):
    w = workloads.WORKLOADS[name]
    prob = TPProblem.build(w.irreps_in, w.sh_lmax, w.irreps_out)
    d = workloads.make_inputs(w, len(prob.paths), prob.weight_numel)
    d.update(workloads.make_cotangents(w, len(d["src"]), prob.weight_numel))
    return w, prob, d


@pytest.mark.parametrize("name", ["tiny", "c1k"])
def test_workload_full(tp, name):
    w, prob, d = workload_inputs(name)
    spec = (w.irreps_in, w.sh_lmax, w.irreps_out, w.dtype)
    args = (d["x"], d["Y"], d["W"], d["G"], d["ggx"], d["ggY"], d["ggW"])
    log(f"[dd] workload {name} N={d['n_nodes']} E={len(d['src'])}")
    got = run_dd(tp, spec, d["n_nodes"], d["src"], d["dst"], *args)
    ref = tp_double_backward(prob, *args, d["src"], d["dst"], d["n_nodes"])
    check(got, ref, w.dtype, f"workload {name}")


@pytest.mark.parametrize("name,n_rows,n_edges", [("c4k", 160, 2500), ("c2k", 160, 2500), ("c28k", 64, 1000)])
def test_workload_sampled(tp, name, n_rows, n_edges):
    import torch
    w, prob, d = workload_inputs(name)
    N, src, dst = d["n_nodes"], d["src"], d["dst"]
    E = len(src)
    spec = (w.irreps_in, w.sh_lmax, w.irreps_out, w.dtype)
    log(f"[dd] workload {name} sampled N={N} E={E}")
    gx, gY, gW, gG = run_dd(tp, spec, N, src, dst, d["x"], d["Y"], d["W"], d["G"], d["ggx"], d["ggY"], d["ggW"])
    torch.cuda.empty_cache()
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([rng.choice(N, n_rows, replace=False), [0, N - 1]]))
    t0 = time.time()

    def oracle(m):
        return tp_double_backward(prob, d["x"], d["Y"][m], d["W"][m], d["G"], d["ggx"], d["ggY"][m], d["ggW"][m],
                                  src[m], dst[m], N)

    r = oracle(np.isin(dst, rows))           # every in-edge of the chosen destinations
    e_gG = rel_err(gG[rows], r[3][rows])
    r = oracle(np.isin(src, rows))           # every out-edge of the chosen sources
    e_gx = rel_err(gx[rows], r[0][rows])
    es = np.unique(np.concatenate([rng.choice(E, n_edges, replace=False), [0, E - 1]]))
    r = oracle(es)
    errs = dict(grad_x=e_gx, grad_Y=rel_err(gY[es], r[1]), grad_W=rel_err(gW[es], r[2]), grad_G=e_gG)
    log(f"[dd] workload {name} sampled errors {errs} (oracle {time.time() - t0:.1f}s)")
    for k, v in errs.items():
        assert v <= TOL[w.dtype], (name, k, v)


# ----------------------------------------------------------------- edge cases
SPEC_C = ("8x0e+8x1o+8x2e", 2, "8x0e+8x1o+8x2e", "f64")


def small_graph(rng, n, p):
    a = rng.random((n, n)) < p
    np.fill_diagonal(a, False)
    dst, src = np.nonzero(a)
    return src.astype(np.int32), dst.astype(np.int32)


@pytest.mark.parametrize("drop", [(), ("a",), ("b",), ("c",), ("a", "b"), ("b", "c"), ("a", "c"), ("a", "b", "c")])
def test_null_cotangents(tp, drop):
    rng = np.random.default_rng(31)
    src, dst = small_graph(rng, 33, 0.25)
    got = check_full(tp, SPEC_C, 33, src, dst, seed=2, label="null", drop=drop)
    if len(drop) == 3:
        assert all(np.all(t == 0) for t in got)


def test_empty_graph(tp):
    src = dst = np.zeros(0, np.int32)
    gx, gY, gW, gG = check_full(tp, SPEC_C, 6, src, dst, label="empty")
    assert np.all(gx == 0) and np.all(gG == 0) and gY.shape[0] == 0 and gW.shape[0] == 0


def test_self_loops_isolated_duplicates_shuffled(tp):
    check_full(tp, SPEC_C, 1, np.zeros(5, np.int32), np.zeros(5, np.int32), label="self-loops")
    rng = np.random.default_rng(32)
    src, dst = small_graph(rng, 40, 0.2)
    keep = (dst != 7) & (src != 9)
    src, dst = src[keep], dst[keep]
    src = np.concatenate([src, src[:30]])
    dst = np.concatenate([dst, dst[:30]])
    perm = rng.permutation(len(src))
    gx, _, _, gG = check_full(tp, SPEC_C, 41, src[perm], dst[perm], label="shuffled")
    assert np.all(gG[7] == 0) and np.all(gx[9] == 0) and np.all(gG[40] == 0) and np.all(gx[40] == 0)


def test_hub_node(tp):
    rng = np.random.default_rng(33)
    n = 1200
    src = np.concatenate([np.arange(1, n), rng.integers(0, n, 400), np.zeros(900, np.int64)]).astype(np.int32)
    dst = np.concatenate([np.zeros(n - 1, np.int64), rng.integers(0, n, 400),
                          rng.integers(0, n, 900)]).astype(np.int32)
    check_full(tp, ("16x0e+16x1o+16x2e+16x3o", 3, "16x0e+16x1o+16x2e+16x3o", "f32"), n, src, dst, label="hub")


@pytest.mark.parametrize("spec", [
    ("8x1o+8x0e", 2, "8x1e+8x2o+8x0o", "f64"),                        # odd l1+l2+l3 paths
    ("4x0e+4x1e", 1, "4x0o+4x1o+4x2o", "f64"),                       # even and odd paths mixed
    ("24x0e+24x1o+24x2e", 2, "24x0e+24x1o+24x2e", "f32"),             # U not a power of two
    ("1x0e+1x1o+1x2e+1x3o", 3, "1x0e+1x1o+1x2e+1x3o", "f64"),         # U = 1
    ("64x0e+64x1o+64x2e", 2, "64x0e+64x1o+64x2e", "f64"),             # U = 64
    ("6x0e+6x2e", 1, "6x1o+6x2e+6x3o", "f32"),                        # missing l, SH below the bound
    ("16x0e", 0, "16x0e", "f32"),                                     # scalars only
    ("32x0e+32x1o+32x2e+32x3o", 3, "32x0e+32x1o+32x2e+32x3o", "f32"),  # the 4096-atom irreps, full plan
    ("8x0e+8x1o+8x2e+8x3o+8x4e", 4, "8x0e+8x1o+8x2e+8x3o+8x4e", "f32"),
    ("8x4e+8x1o", 3, "8x3o+8x0e+8x4e", "f64"),
])
def test_irreps_variants(tp, spec):
    rng = np.random.default_rng(zlib.crc32(repr(spec).encode()))
    src, dst = small_graph(rng, 37, 0.25)
    check_full(tp, spec, 37, src, dst, seed=3, label="variant")


@pytest.mark.parametrize("spec", [
    ("8x0e+8x1o+8x1e+8x2e", 2, "8x0e+8x0o+8x1o+8x1e+8x2e+8x2o", "f32"),
    ("16x1e+16x0e+16x1o", 1, "16x1o+16x1e", "f64"),
    ("8x2o+8x2e", 1, "8x1e+8x2e", "f64"),
])
def test_both_parities_of_one_l(tp, spec):
    """Plans with both parities of some l (passes by segment type, the later
    adding into grad_G, grad_x and grad_Y) against the oracle."""
    rng = np.random.default_rng(zlib.crc32(repr(spec).encode()) + 1)
    src, dst = small_graph(rng, 41, 0.2)
    check_full(tp, spec, 41, src, dst, seed=5, label="both-parities")


def test_partial_outputs(tp):
    rng = np.random.default_rng(34)
    src, dst = small_graph(rng, 30, 0.3)
    prob, x, Y, W, G, a, b, c = random_case(SPEC_C, 30, src, dst, 4)
    ref = tp_double_backward(prob, x, Y, W, G, a, b, c, src, dst, 30)
    for need in ((True, False, False, False), (False, True, False, False), (False, False, True, False),
                 (False, False, False, True), (False, True, True, True)):
        got = run_dd(tp, SPEC_C, 30, src, dst, x, Y, W, G, a, b, c, need=need)
        for flag, u, v in zip(need, got, ref):
            if flag:
                assert rel_err(u, v) <= 1e-11
            else:
                assert u is None
    # grad_out may be omitted when only grad_G is wanted
    import torch
    plan = tp.tpconv_plan(*SPEC_C)
    t = lambda v: torch.from_numpy(np.ascontiguousarray(v)).cuda()  # noqa: E731
    g = tp.tpconv_graph_create(30, t(src.astype(np.int32)), t(dst.astype(np.int32)))
    outs = tp.tpconv_double_backward(plan, g, t(x), t(Y), t(W), None, t(a), t(b), t(c),
                                     need=(False, False, False, True))
    assert rel_err(outs[3].cpu().numpy(), ref[3]) <= 1e-11
    with pytest.raises(tp.TPConvError):
        tp.tpconv_double_backward(plan, g, t(x), t(Y), t(W), None, t(a), t(b), t(c))


def test_bitwise_deterministic(tp):
    w, prob, d = workload_inputs("c1k")
    spec = (w.irreps_in, w.sh_lmax, w.irreps_out, w.dtype)
    args = (d["x"], d["Y"], d["W"], d["G"], d["ggx"], d["ggY"], d["ggW"])
    u = run_dd(tp, spec, d["n_nodes"], d["src"], d["dst"], *args)
    v = run_dd(tp, spec, d["n_nodes"], d["src"], d["dst"], *args)
    for p, q in zip(u, v):
        assert np.array_equal(p, q)
