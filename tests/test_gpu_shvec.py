"""GPU parity of the convolution with the harmonics evaluated inside its kernels
(tpconv_forward_vec, tpconv_backward_vec), through the C ABI, against the fp64
oracle's chain: Y = sh_edges(vec), tp_forward / tp_backward on that Y, and
grad_vec = sh_backward(vec, dY), grad_pos = positions_backward(grad_vec).

Metric as elsewhere: max |T_gpu - T_ref| / rms(T_ref) per tensor, <= 1e-5
(fp32) or 1e-11 (fp64).  The edge vectors are cast to the plan's dtype and the
oracle consumes the cast values; the kernels round Y to the dtype once, which
the fp32 bar absorbs (Y's rounding moves the outputs by ~1e-7 of their RMS).
Small graphs compare every element; the full-size workloads compare sampled
rows and edges, each computed exactly by the oracle from the edges feeding it.
The graphs include rows longer than one chunk of staged edges (32 edges in the
forward, 64 in the backward) and zero vectors.
"""

import sys

import numpy as np
import pytest

import workloads
from oracle import TPProblem, positions_backward, sh_backward, sh_edges, tp_backward, tp_forward

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f64": 1e-11}


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


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_vec(tp, spec, n_nodes, src, dst, x, vec, W, G):
    """Fused path: (out, grad_x, grad_vec, grad_W, grad_pos); and the three-kernel chain's
    (out, grad_vec) on the same inputs."""
    import torch
    plan = tp.tpconv_plan(*spec)
    g = tp.tpconv_graph_create(n_nodes, dev(np.asarray(src, np.int32)), dev(np.asarray(dst, np.int32)))
    xt, vt, Wt, Gt = dev(x), dev(vec), dev(W), dev(G)
    out = tp.tpconv_forward_vec(plan, g, xt, vt, Wt)
    dx, gv, dW = tp.tpconv_backward_vec(plan, g, xt, vt, Wt, Gt)
    gp = tp.tpconv_positions_backward(plan, g, gv)
    Y = tp.tpconv_sh(plan, vt)
    out3 = tp.tpconv_forward(plan, g, xt, Y, Wt)
    _, dY3, _ = tp.tpconv_backward(plan, g, xt, Y, Wt, Gt, need=(False, True, False))
    gv3 = tp.tpconv_sh_backward(plan, vt, dY3)
    torch.cuda.synchronize()
    c = lambda a: a.cpu().numpy()  # noqa: E731
    return c(out), c(dx), c(gv), c(dW), c(gp), c(out3), c(gv3)


def check_all(tp, spec, n_nodes, src, dst, x, vec, W, G, label):
    prob = TPProblem.build(spec[0], spec[1], spec[2])
    lsh, dt = spec[1], spec[3]
    log(f"[shvec] {label} spec={spec} N={n_nodes} E={len(src)}")
    out, dx, gv, dW, gp, out3, gv3 = run_vec(tp, spec, n_nodes, src, dst, x, vec, W, G)
    rY = sh_edges(lsh, vec) if len(src) else np.zeros((0, (lsh + 1) ** 2))
    r_out = tp_forward(prob, x, rY, W, src, dst, n_nodes)
    r_dx, r_dY, r_dW = tp_backward(prob, x, rY, W, G, src, dst, n_nodes)
    r_gv = sh_backward(lsh, vec, r_dY) if len(src) else np.zeros((0, 3))
    r_gp = positions_backward(r_gv, src, dst, n_nodes)
    errs = dict(out=rel_err(out, r_out), dx=rel_err(dx, r_dx), dW=rel_err(dW, r_dW), grad_vec=rel_err(gv, r_gv),
                grad_pos=rel_err(gp, r_gp))
    log(f"[shvec] {label} errors {errs}; fused vs three kernels: out {rel_err(out, out3):.2e}, "
        f"grad_vec {rel_err(gv, gv3):.2e}")
    for k, v in errs.items():
        assert v <= TOL[dt], (label, k, v)
    return out, dx, gv, dW, gp


def random_inputs(spec, n_nodes, src, dst, seed):
    prob = TPProblem.build(spec[0], spec[1], spec[2])
    npdt = np.float32 if spec[3] == "f32" else np.float64
    rng = np.random.default_rng(seed)
    E = len(src)
    x = rng.standard_normal((n_nodes, prob.dim_in)).astype(npdt)
    vec = (rng.standard_normal((E, 3)) * rng.uniform(0.5, 5.0, (E, 1))).astype(npdt)
    W = (rng.standard_normal((E, prob.weight_numel)) / np.sqrt(len(prob.paths))).astype(npdt)
    G = rng.standard_normal((n_nodes, prob.dim_out)).astype(npdt)
    return x, vec, W, G


def hub_graph(rng, n, e_rand, hub_in, hub_out):
    """Random edges plus node 0 with hub_in in-edges and hub_out out-edges, in shuffled order."""
    src = np.concatenate([rng.integers(0, n, e_rand), rng.integers(1, n, hub_in), np.zeros(hub_out, np.int64)])
    dst = np.concatenate([rng.integers(0, n, e_rand), np.zeros(hub_in, np.int64), rng.integers(1, n, hub_out)])
    perm = rng.permutation(len(src))
    return src[perm].astype(np.int32), dst[perm].astype(np.int32)


def irreps(mul, L):
    return "+".join(f"{mul}x{l}{'e' if l % 2 == 0 else 'o'}" for l in range(L + 1))


# (mul, L, dtype, nodes): nodes > 1024 runs whole rows per wavefront, fewer splits rows over a block
CASES = [(32, 3, "f32", 1500), (32, 3, "f32", 300), (16, 3, "f32", 1300), (64, 1, "f64", 1100),
         (64, 2, "f32", 200), (16, 4, "f64", 1200), (32, 4, "f64", 250), (16, 4, "f32", 1100), (32, 0, "f32", 1100),
         (16, 1, "f64", 90)]


@pytest.mark.parametrize("mul,L,dt,n", CASES)
def test_random_graph_with_hub(tp, mul, L, dt, n):
    rng = np.random.default_rng(1000 * L + mul + n)
    src, dst = hub_graph(rng, n, 6 * n, hub_in=700, hub_out=333)
    spec = (irreps(mul, L), L, irreps(mul, L), dt)
    x, vec, W, G = random_inputs(spec, n, src, dst, seed=n + L)
    vec[::53] = 0.0                                   # zero vectors: Y = (1, 0, ...), no gradient
    vec[1] = [0.0, 0.0, 1.5]                          # along the axes
    vec[2] = [0.0, -2.0, 0.0]
    _, _, gv, _, _ = check_all(tp, spec, n, src, dst, x, vec, W, G, label=f"U={mul} L={L} {dt} N={n} hub")
    assert np.all(gv[::53] == 0.0)


# plans run by the kernels with a run-time path table: U not a power of two,
# SH bound below or above the segments' l, odd paths, unsorted segments
RT_SPECS = [("5x0e+5x1o+5x2e", 2, "5x0e+5x1o+5x2e", "f32"), ("8x0e+8x1o+8x2e", 1, "8x0e+8x1o+8x2e", "f64"),
            ("3x1o+3x0e", 2, "3x1e+3x2o+3x0o", "f64"), ("4x0e+4x1o", 3, "4x0e+4x1o+4x2e+4x3o", "f32"),
            ("1x0e+1x1o+1x2e+1x3o+1x4e", 4, "1x0e+1x1o+1x2e+1x3o+1x4e", "f64")]


@pytest.mark.parametrize("spec", RT_SPECS)
def test_run_time_plans(tp, spec):
    rng = np.random.default_rng(7)
    n = 400
    src, dst = hub_graph(rng, n, 5 * n, hub_in=150, hub_out=90)
    x, vec, W, G = random_inputs(spec, n, src, dst, seed=8)
    vec[::41] = 0.0
    check_all(tp, spec, n, src, dst, x, vec, W, G, label=f"run-time plan {spec}")


@pytest.mark.parametrize("name", ["tiny", "c1k"])
def test_workload_full(tp, name):
    w = workloads.WORKLOADS[name]
    prob = TPProblem.build(w.irreps_in, w.sh_lmax, w.irreps_out)
    d = workloads.make_inputs(w, len(prob.paths), prob.weight_numel)
    spec = (w.irreps_in, w.sh_lmax, w.irreps_out, w.dtype)
    check_all(tp, spec, d["n_nodes"], d["src"], d["dst"], d["x"], d["vec"].astype(w.np_dtype), d["W"], d["G"],
              label=name)


@pytest.mark.parametrize("name,n_rows,n_edges", [("c4k", 120, 2000), ("c2k", 120, 2000), ("c28k", 64, 1200)])
def test_workload_sampled(tp, name, n_rows, n_edges):
    """Full-size run; sampled destination rows (out), source rows (dx) and edges (dW, grad_vec)."""
    w = workloads.WORKLOADS[name]
    prob = TPProblem.build(w.irreps_in, w.sh_lmax, w.irreps_out)
    d = workloads.make_inputs(w, len(prob.paths), prob.weight_numel)
    N, src, dst = d["n_nodes"], d["src"], d["dst"]
    E = len(src)
    vec = d["vec"].astype(w.np_dtype)
    spec = (w.irreps_in, w.sh_lmax, w.irreps_out, w.dtype)
    log(f"[shvec] workload {name} sampled N={N} E={E}")
    out, dx, gv, dW, _, out3, gv3 = run_vec(tp, spec, N, src, dst, d["x"], vec, d["W"], d["G"])
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([rng.choice(N, n_rows, replace=False), [0, N - 1]]))
    m = np.isin(dst, rows)
    r_out = tp_forward(prob, d["x"], sh_edges(w.sh_lmax, vec[m]), d["W"][m], src[m], dst[m], N)
    m = np.isin(src, rows)
    r_dx, _, _ = tp_backward(prob, d["x"], sh_edges(w.sh_lmax, vec[m]), d["W"][m], d["G"], src[m], dst[m], N)
    es = np.unique(np.concatenate([rng.choice(E, n_edges, replace=False), [0, E - 1]]))
    _, r_dY, r_dW = tp_backward(prob, d["x"], sh_edges(w.sh_lmax, vec[es]), d["W"][es], d["G"], src[es], dst[es], N)
    r_gv = sh_backward(w.sh_lmax, vec[es], r_dY)
    errs = dict(out=rel_err(out[rows], r_out[rows]), dx=rel_err(dx[rows], r_dx[rows]), dW=rel_err(dW[es], r_dW),
                grad_vec=rel_err(gv[es], r_gv))
    log(f"[shvec] workload {name} sampled errors {errs}; fused vs three kernels over all edges: "
        f"out {rel_err(out, out3):.2e}, grad_vec {rel_err(gv, gv3):.2e}")
    for k, v in errs.items():
        assert v <= TOL[w.dtype], (name, k, v)


def test_empty_graph_and_unsupported_plan(tp):
    import torch
    spec = (irreps(16, 2), 2, irreps(16, 2), "f64")
    e = np.zeros(0, np.int32)
    x, vec, W, G = random_inputs(spec, 7, e, e, seed=1)
    out, dx, gv, dW, gp = check_all(tp, spec, 7, e, e, x, vec, W, G, label="empty")
    assert np.all(out == 0) and np.all(dx == 0) and gv.shape == (0, 3) and np.all(gp == 0)
    # a plan the fused kernels do not cover (both parities of l = 1: several passes) is refused
    plan = tp.tpconv_plan("16x0e+16x1o+16x1e", 1, "16x0e+16x1o+16x1e", "f32")
    rng = np.random.default_rng(2)
    src = rng.integers(0, 10, 40).astype(np.int32)
    g = tp.tpconv_graph_create(10, dev(src), dev(src[::-1].copy()))
    xt = torch.zeros((10, plan.dim_in), dtype=torch.float32, device="cuda")
    vt = torch.ones((40, 3), dtype=torch.float32, device="cuda")
    Wt = torch.zeros((40, plan.weight_numel), dtype=torch.float32, device="cuda")
    with pytest.raises(tp.TPConvError) as ei:
        tp.tpconv_forward_vec(plan, g, xt, vt, Wt)
    assert ei.value.name == "TPCONV_E_UNSUPPORTED"
    with pytest.raises(tp.TPConvError) as ei:
        tp.tpconv_backward_vec(plan, g, xt, vt, Wt, torch.zeros_like(xt))
    assert ei.value.name == "TPCONV_E_UNSUPPORTED"


def test_force_chain_c4k_sampled(tp):
    """Forces of the energy <G, out(x, Y(vec), W)> on c4k through the fused backward and
    tpconv_positions_backward, at sampled atoms: each sampled atom's force needs grad_vec of
    every edge touching it, which the oracle computes for those edges only."""
    import torch
    w = workloads.WORKLOADS["c4k"]
    prob = TPProblem.build(w.irreps_in, w.sh_lmax, w.irreps_out)
    d = workloads.make_inputs(w, len(prob.paths), prob.weight_numel)
    N, src, dst = d["n_nodes"], d["src"], d["dst"]
    vec = d["vec"].astype(w.np_dtype)
    plan = tp.tpconv_plan(w.irreps_in, w.sh_lmax, w.irreps_out, w.dtype)
    g = tp.tpconv_graph_create(N, dev(src), dev(dst))
    _, gv, _ = tp.tpconv_backward_vec(plan, g, dev(d["x"]), dev(vec), dev(d["W"]), dev(d["G"]),
                                      need=(False, True, False))
    gp = tp.tpconv_positions_backward(plan, g, gv).cpu().numpy()
    torch.cuda.synchronize()
    rng = np.random.default_rng(12)
    atoms = np.unique(np.concatenate([rng.choice(N, 60, replace=False), [0, N - 1]]))
    m = np.isin(src, atoms) | np.isin(dst, atoms)
    _, r_dY, _ = tp_backward(prob, d["x"], sh_edges(w.sh_lmax, vec[m]), d["W"][m], d["G"], src[m], dst[m], N)
    r_gp = positions_backward(sh_backward(w.sh_lmax, vec[m], r_dY), src[m], dst[m], N)
    err = rel_err(gp[atoms], r_gp[atoms])
    log(f"[shvec] c4k force chain at {len(atoms)} atoms ({int(m.sum())} edges): grad_pos error {err:.3e}")
    assert err <= TOL[w.dtype]
