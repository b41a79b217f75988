"""The allocation-free SO(2) backward (tpconv_so2_backward_noalloc) against the
workspace entry point (tpconv_so2_backward), through the C ABI.

Two calls in a row on one device share the library's scratch: the 4096-atom
graph (l <= 3, 32 channels, 214 648 edges; fewer blocks of edges fit the
scratch than the workspace entry point uses) and then the 1024-atom graph
(l <= 2, 32 channels).  grad_x comes from the same kernels and must be
bitwise equal; grad_weights sums its blocks of edges differently and must
agree to the fp32 bar (max |diff| / rms <= 1e-5).  Neither call allocates
device memory (outputs are given).
"""

import sys

import numpy as np
import pytest

import workloads
from oracle.so2 import weight_numel

pytestmark = pytest.mark.gpu

TOL = 1e-5


def log(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def tp():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
    from equivariant_mlip_tensor_amd import tpconv
    return tpconv


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / np.sqrt(np.mean(b ** 2)))


def test_noalloc_matches_workspace_entry_point(tp):
    import torch
    cases = []
    for name in ("c4k", "c1k"):                      # the second call is the smaller one
        w = workloads.WORKLOADS[name]
        lmax, C = workloads.SO2_SHAPES[name]
        inp = workloads.make_so2_inputs(w, weight_numel(lmax, C))
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
        g = tp.tpconv_graph_create(inp["n_nodes"], dev(inp["src"]), dev(inp["dst"]))
        D = tp.tpconv_so2_rotations(lmax, dev(inp["vec"].astype(np.float32)))
        x, wt, G = dev(inp["x"]), dev(inp["weights"]), dev(inp["G"])
        ref_x, ref_w = tp.tpconv_so2_backward(g, lmax, C, x, D, wt, G)
        cases.append((name, lmax, C, g, D, x, wt, G, ref_x, ref_w))
    torch.cuda.synchronize()
    outs = []
    for name, lmax, C, g, D, x, wt, G, _, ref_w in cases:
        gx = torch.full_like(x, float("nan"))
        gw = torch.full_like(ref_w, float("nan"))
        outs.append((gx, gw))
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    for (name, lmax, C, g, D, x, wt, G, _, _), (gx, gw) in zip(cases, outs):
        log(f"[noalloc] {name} l<={lmax} C={C} E={g.n_edges}")
        tp.tpconv_so2_backward_noalloc(g, lmax, C, x, D, wt, G, gx, gw)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    for (name, _, _, _, _, _, _, _, ref_x, ref_w), (gx, gw) in zip(cases, outs):
        assert torch.equal(gx, ref_x), name
        err = rel_err(gw.cpu().numpy(), ref_w.cpu().numpy())
        log(f"[noalloc] {name} grad_weights vs workspace entry point {err:.3e}")
        assert err <= TOL, (name, err)
    # only one of the outputs
    name, lmax, C, g, D, x, wt, G, ref_x, ref_w = cases[1]
    gw = torch.zeros_like(ref_w)
    tp.tpconv_so2_backward_noalloc(g, lmax, C, x, D, wt, G, None, gw)
    torch.cuda.synchronize()
    assert rel_err(gw.cpu().numpy(), ref_w.cpu().numpy()) <= TOL
