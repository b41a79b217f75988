"""GPU parity of the upstream step: edge harmonics (tpconv_sh), their gradient
(tpconv_sh_backward) and the position gradient (tpconv_positions_backward),
through the C ABI, against the fp64 oracle; and the whole force chain
forward -> backward -> sh_backward -> positions_backward.

Metric as elsewhere: max |T_gpu - T_ref| / rms(T_ref) per tensor, <= 1e-5
(fp32) or 1e-11 (fp64).  Edge vectors come from the workloads' own
geometry (minimum-image vectors of the periodic boxes), cast to the
workload's dtype; the oracle consumes the cast values.
"""

import sys

import numpy as np
import pytest

import workloads
from oracle import TPProblem, positions_backward, sh_backward, sh_edges, tp_backward

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


def run_upstream(tp, spec, n_nodes, src, dst, vec, gY):
    import torch
    plan = tp.tpconv_plan(*spec)
    g = tp.tpconv_graph_create(n_nodes, dev(np.asarray(src, np.int32)), dev(np.asarray(dst, np.int32)))
    v = dev(vec)
    Y = tp.tpconv_sh(plan, v)
    gv = tp.tpconv_sh_backward(plan, v, dev(gY))
    gp = tp.tpconv_positions_backward(plan, g, gv)
    torch.cuda.synchronize()
    return Y.cpu().numpy(), gv.cpu().numpy(), gp.cpu().numpy()


def check_upstream(tp, spec, n_nodes, src, dst, vec, seed, label):
    dt = spec[3]
    npdt = np.float32 if dt == "f32" else np.float64
    lsh = spec[1]
    rng = np.random.default_rng(seed)
    vec = np.asarray(vec).astype(npdt)
    gY = rng.standard_normal((len(src), (lsh + 1) ** 2)).astype(npdt)
    Y, gv, gp = run_upstream(tp, spec, n_nodes, src, dst, vec, gY)
    rY = sh_edges(lsh, vec)
    rgv = sh_backward(lsh, vec, gY)
    rgp = positions_backward(gv.astype(np.float64), src, dst, n_nodes)   # the reduction alone, on the GPU's input
    rgp_chain = positions_backward(rgv, src, dst, n_nodes)
    errs = dict(Y=rel_err(Y, rY), grad_vec=rel_err(gv, rgv), grad_pos=rel_err(gp, rgp),
                grad_pos_chain=rel_err(gp, rgp_chain))
    log(f"[forces] {label} spec={spec} N={n_nodes} E={len(src)} errors {errs}")
    for k, v in errs.items():
        assert v <= TOL[dt], (label, k, v)
    return Y, gv, gp


@pytest.mark.parametrize("name", ["tiny", "c1k", "c4k", "c2k", "c28k"])
def test_workload_geometry(tp, name):
    w = workloads.WORKLOADS[name]
    g = workloads.make_graph(w)
    spec = (w.irreps_in, w.sh_lmax, w.irreps_out, w.dtype)
    check_upstream(tp, spec, w.n_atoms, g["src"], g["dst"], g["vec"], seed=w.key, label=name)


@pytest.mark.parametrize("lsh,dt", [(0, "f32"), (1, "f64"), (2, "f32"), (3, "f64"), (4, "f32"), (4, "f64")])
def test_every_l_bound_and_zero_vectors(tp, lsh, dt):
    rng = np.random.default_rng(70 + lsh)
    n, E = 50, 700
    src = rng.integers(0, n, E).astype(np.int32)
    dst = rng.integers(0, n, E).astype(np.int32)
    vec = rng.standard_normal((E, 3)) * rng.uniform(0.05, 6.0, (E, 1))
    vec[::97] = 0.0                                  # zero vectors: Y = (1, 0, ...), no gradient
    vec[5] = [0.0, 0.0, 2.0]                         # along the axes
    vec[6] = [0.0, -3.0, 0.0]
    vec[7] = [1e-3, 0.0, 0.0]                        # short
    spec = ("4x0e", lsh, "4x0e", dt)
    Y, gv, _ = check_upstream(tp, spec, n, src, dst, vec, seed=lsh, label=f"l<={lsh} {dt}")
    assert np.all(Y[::97, 0] == 1.0) and np.all(Y[::97, 1:] == 0.0) and np.all(gv[::97] == 0.0)


def test_empty_and_isolated_and_hub(tp):
    spec = ("4x0e+4x1o", 2, "4x0e+4x1o", "f64")
    e = np.zeros(0, np.int32)
    Y, gv, gp = run_upstream(tp, spec, 5, e, e, np.zeros((0, 3)), np.zeros((0, 9)))
    assert Y.shape == (0, 9) and gv.shape == (0, 3) and np.all(gp == 0.0)
    rng = np.random.default_rng(71)
    n = 900
    src = np.concatenate([np.arange(1, n), rng.integers(0, n, 300)]).astype(np.int32)
    dst = np.concatenate([np.zeros(n - 1, np.int32), rng.integers(0, n, 300)]).astype(np.int32)
    keep = (src != 17) & (dst != 17)                 # node 17: no edges at all
    src, dst = src[keep], dst[keep]
    vec = rng.standard_normal((len(src), 3))
    _, _, gp = check_upstream(tp, ("8x0e+8x1o", 3, "8x0e+8x1o", "f32"), n, src, dst, vec, seed=3, label="hub")
    assert np.all(gp[17] == 0.0)


@pytest.mark.parametrize("name", ["tiny", "c1k"])
def test_force_chain(tp, name):
    """Energy <G, out(x, Y(vec), W)>: its position gradient from the GPU chain
    (sh -> forward/backward -> sh_backward -> positions_backward) against the
    oracle's chain on the same inputs."""
    import torch
    w = workloads.WORKLOADS[name]
    prob = TPProblem.build(w.irreps_in, w.sh_lmax, w.irreps_out)
    d = workloads.make_inputs(w, len(prob.paths), prob.weight_numel)
    npdt = w.np_dtype
    vec = d["vec"].astype(npdt)
    plan = tp.tpconv_plan(w.irreps_in, w.sh_lmax, w.irreps_out, w.dtype)
    g = tp.tpconv_graph_create(d["n_nodes"], dev(d["src"]), dev(d["dst"]))
    v = dev(vec)
    Y = tp.tpconv_sh(plan, v)
    _, dY, _ = tp.tpconv_backward(plan, g, dev(d["x"]), Y, dev(d["W"]), dev(d["G"]), need=(False, True, False))
    gpos = tp.tpconv_positions_backward(plan, g, tp.tpconv_sh_backward(plan, v, dY))
    torch.cuda.synchronize()
    rY = sh_edges(w.sh_lmax, vec)
    _, rdY, _ = tp_backward(prob, d["x"], rY, d["W"], d["G"], d["src"], d["dst"], d["n_nodes"])
    ref = positions_backward(sh_backward(w.sh_lmax, vec, rdY), d["src"], d["dst"], d["n_nodes"])
    err = rel_err(gpos.cpu().numpy(), ref)
    log(f"[forces] chain {name} grad_pos error {err:.3e}")
    assert err <= TOL[w.dtype]
    # internal forces sum to zero (every edge adds to one atom what it takes from another)
    gp = gpos.cpu().numpy().astype(np.float64)
    assert np.abs(gp.sum(axis=0)).max() <= 1e-5 * np.abs(gp).sum()


def test_force_chain_c4k_sampled(tp):
    """The three-kernel force chain (tpconv_sh -> tpconv_backward -> tpconv_sh_backward ->
    tpconv_positions_backward) on the full 4096-atom workload, checked at sampled atoms: each
    sampled atom's force needs grad_vec of every edge touching it, which the oracle computes
    for those edges only."""
    import torch
    w = workloads.WORKLOADS["c4k"]
    prob = TPProblem.build(w.irreps_in, w.sh_lmax, w.irreps_out)
    d = workloads.make_inputs(w, len(prob.paths), prob.weight_numel)
    N, src, dst = d["n_nodes"], d["src"], d["dst"]
    vec = d["vec"].astype(w.np_dtype)
    plan = tp.tpconv_plan(w.irreps_in, w.sh_lmax, w.irreps_out, w.dtype)
    g = tp.tpconv_graph_create(N, dev(src), dev(dst))
    v = dev(vec)
    Y = tp.tpconv_sh(plan, v)
    _, dY, _ = tp.tpconv_backward(plan, g, dev(d["x"]), Y, dev(d["W"]), dev(d["G"]), need=(False, True, False))
    gpos = tp.tpconv_positions_backward(plan, g, tp.tpconv_sh_backward(plan, v, dY)).cpu().numpy()
    torch.cuda.synchronize()
    rng = np.random.default_rng(13)
    atoms = np.unique(np.concatenate([rng.choice(N, 60, replace=False), [0, N - 1]]))
    m = np.isin(src, atoms) | np.isin(dst, atoms)
    _, rdY, _ = tp_backward(prob, d["x"], sh_edges(w.sh_lmax, vec[m]), d["W"][m], d["G"], src[m], dst[m], N)
    ref = positions_backward(sh_backward(w.sh_lmax, vec[m], rdY), src[m], dst[m], N)
    err = rel_err(gpos[atoms], ref[atoms])
    log(f"[forces] chain c4k at {len(atoms)} atoms ({int(m.sum())} edges): grad_pos error {err:.3e}")
    assert err <= TOL[w.dtype]
