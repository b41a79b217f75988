"""Host-side checks of libtpconv.so (CPU only: no kernel is launched).

The library loads, exports every entry point the header declares, and its
host CG-table builder, path list and error paths agree with the oracle and
with the header's contract.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import workloads
from oracle import TPProblem, cg_real

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "equivariant_mlip_tensor_amd", "libtpconv.so")
HEADER = os.path.join(ROOT, "include", "tpconv.h")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libtpconv.so not built")


@pytest.fixture(scope="module")
def tp():
    from equivariant_mlip_tensor_amd import tpconv
    return tpconv


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tpconv_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(tp):
    declared = header_functions()
    assert len(declared) == 32
    assert sorted(tp.EXPORTS) == declared
    lib = ctypes.CDLL(LIB)
    for name in declared:
        assert hasattr(lib, name), name


CASES = [(w.irreps_in, w.sh_lmax, w.irreps_out, w.dtype) for w in workloads.WORKLOADS.values()] + [
    ("3x1o+3x0e", 2, "3x1e+3x2o+3x0o", "f64"),        # odd paths, unsorted segments
    ("5x0e+5x2e", 1, "5x1o+5x2e+5x3o", "f32"),        # missing l, sh below the l bound
    ("1x4e", 4, "1x0e+1x4e", "f64"),
    ("4x0e+4x1o+4x1e+4x2e", 2, "4x0e+4x0o+4x1o+4x1e+4x2e+4x2o", "f32"),   # both parities of one l
    ("2x1e+2x0e+2x1o", 1, "2x1o+2x1e", "f64"),                           # both parities, unsorted
]


@pytest.mark.parametrize("case", CASES)
def test_plan_matches_oracle_paths_and_cg(tp, case):
    irr_in, lsh, irr_out, dt = case
    prob = TPProblem.build(irr_in, lsh, irr_out)
    plan = tp.tpconv_plan(irr_in, lsh, irr_out, dt)
    assert plan.n_paths == len(prob.paths)
    assert plan.weight_numel == prob.weight_numel
    assert (plan.dim_in, plan.dim_out, plan.dim_sh) == (prob.dim_in, prob.dim_out, prob.dim_sh)
    paths = tp.tpconv_plan_paths(plan)
    assert [p[:3] for p in paths] == [tuple(p) for p in prob.paths]
    assert [p[3] for p in paths] == prob.weight_offsets
    entries, ptr, values = tp.tpconv_plan_table(plan)
    assert len(entries) == plan.cg_nnz and ptr[-1] == plan.cg_nnz and len(values) == plan.cg_nvalues
    vals = np.array(values)
    assert np.all(vals > 0)
    # deduplicated: no two stored magnitudes coincide
    assert len(np.unique(np.round(vals, 12))) == len(vals)
    nnz = 0
    for p in range(plan.n_paths):
        l1, l2, l3 = prob.path_ls(p)
        dense = np.zeros((2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1))
        keys = []
        for e in entries[ptr[p]:ptr[p + 1]]:
            m1, m2, m3, neg, vi = e & 15, (e >> 4) & 15, (e >> 8) & 15, (e >> 12) & 1, e >> 13
            dense[m1, m2, m3] = (-1.0 if neg else 1.0) * values[vi]
            keys.append((m1, m2, m3))
        assert keys == sorted(keys)                       # entries ordered by (m1, m2, m3)
        ref = cg_real(l1, l2, l3)
        np.testing.assert_allclose(dense, ref, atol=2e-15, rtol=0)
        assert np.count_nonzero(dense) == np.count_nonzero(ref)   # zeros skipped, none lost
        nnz += np.count_nonzero(ref)
    assert nnz == plan.cg_nnz


def test_workload_path_and_table_sizes(tp):
    # path count, nonzeros and distinct values of the l<=3 and l<=4 workloads
    w3 = workloads.WORKLOADS["c4k"]
    p3 = tp.tpconv_plan(w3.irreps_in, 3, w3.irreps_out, "f32")
    assert (p3.n_paths, p3.cg_nnz, p3.weight_numel) == (23, 353, 736)
    w4 = workloads.WORKLOADS["c2k"]
    p4 = tp.tpconv_plan(w4.irreps_in, 4, w4.irreps_out, "f64")
    assert (p4.n_paths, p4.cg_nnz) == (42, 1158)


@pytest.mark.parametrize("irr_in,lsh,irr_out,dt,status", [
    ("4x1q", 1, "4x1o", "f32", "TPCONV_E_IRREPS"),
    ("4x", 1, "4x1o", "f32", "TPCONV_E_IRREPS"),
    ("", 1, "4x1o", "f32", "TPCONV_E_IRREPS"),
    ("4x1o+", 1, "4x1o", "f32", "TPCONV_E_IRREPS"),
    ("0x1o", 1, "4x1o", "f32", "TPCONV_E_IRREPS"),
    ("4x5e", 1, "4x5e", "f32", "TPCONV_E_UNSUPPORTED"),
    ("4x1o", 5, "4x1o", "f32", "TPCONV_E_UNSUPPORTED"),
    ("4x1o+4x1o", 1, "4x1o", "f32", "TPCONV_E_UNSUPPORTED"),
    ("4x0e", 1, "8x1o", "f32", "TPCONV_E_UNSUPPORTED"),
    ("128x0e", 0, "128x0e", "f32", "TPCONV_E_UNSUPPORTED"),
    ("65x0e+65x1o", 1, "65x0e+65x1o", "f32", "TPCONV_E_UNSUPPORTED"),   # U past one wavefront
    ("64x0e+64x1o", 1, "64x0e", "f32", None),                             # U = 64 is the last one taken
    ("1x0e", 1, "1x2e", "f32", "TPCONV_E_NO_PATHS"),
    ("1x0e", -1, "1x0e", "f32", "TPCONV_E_INVALID_ARG"),
    ("1x0e", 0, "1x0e", 7, "TPCONV_E_INVALID_ARG"),
])
def test_plan_errors(tp, irr_in, lsh, irr_out, dt, status):
    if status is None:
        assert tp.tpconv_plan(irr_in, lsh, irr_out, dt).mul == 64
        return
    with pytest.raises(tp.TPConvError) as ei:
        tp.tpconv_plan(irr_in, lsh, irr_out, dt)
    assert ei.value.name == status
    assert tp.tpconv_last_error()


def test_null_and_size_errors_need_no_gpu(tp):
    lib = tp._lib
    h = ctypes.c_void_p()
    assert lib.tpconv_plan(None, 1, b"1x0e", 0, ctypes.byref(h)) == 1
    assert lib.tpconv_plan(b"1x0e", 1, b"1x0e", 0, None) == 1
    assert lib.tpconv_plan_query(None, None) == 1
    assert lib.tpconv_forward(None, None, None, None, None, None, None) == 1
    assert lib.tpconv_backward(None, None, None, None, None, None, None, None, None, None) == 1
    assert lib.tpconv_forward_vec(None, None, None, None, None, None, None) == 1
    assert lib.tpconv_backward_vec(None, None, None, None, None, None, None, None, None, None) == 1
    assert lib.tpconv_double_backward(*([None] * 14)) == 1
    assert lib.tpconv_sh(None, 0, None, None, None) == 1
    assert lib.tpconv_sh_backward(None, 0, None, None, None, None) == 1
    assert lib.tpconv_positions_backward(None, None, None, None, None) == 1
    assert lib.tpconv_graph_workspace_bytes(-1, 5) == 0
    ws = tp.tpconv_graph_workspace_bytes(10, 100)
    assert ws >= 4 * (2 * 11 + 4 * 100 + 2 * 10 + 1)
    g = ctypes.c_void_p()
    buf = (ctypes.c_uint8 * 64)()
    # errors detected before anything is launched
    assert lib.tpconv_graph_create(-1, 0, None, None, buf, 64, None, ctypes.byref(g)) == 1
    assert lib.tpconv_graph_create(10, 1 << 31, buf, buf, buf, 64, None, ctypes.byref(g)) == 1
    assert lib.tpconv_graph_create(10, 5, None, None, buf, 64, None, ctypes.byref(g)) == 1
    assert lib.tpconv_graph_create(10, 100, buf, buf, buf, 64, None, ctypes.byref(g)) == 5
    assert "workspace" in tp.tpconv_last_error()


def test_so2_sizes_and_errors_need_no_gpu(tp):
    from oracle.so2 import weight_numel
    lib = tp._lib
    for L in (1, 2, 3):
        for C in (16, 32):
            assert tp.tpconv_so2_weight_numel(L, C) == weight_numel(L, C)
            nb = min(512, max(1, -(-100000 // 64)))
            assert tp.tpconv_so2_workspace_bytes(L, C, 100000) == (nb + 1) * weight_numel(L, C) * 4
    assert tp.tpconv_so2_weight_numel(3, 32) == 45056
    for L, C in ((0, 16), (4, 16), (3, 8), (3, 64), (2, 24)):
        assert tp.tpconv_so2_weight_numel(L, C) == 0
        assert tp.tpconv_so2_workspace_bytes(L, C, 10) == 0
    buf = (ctypes.c_uint8 * 64)()
    assert lib.tpconv_so2_rotations(5, 0, 1, buf, buf, None) == 3
    assert lib.tpconv_so2_rotations(2, 0, 1, None, None, None) == 1
    assert lib.tpconv_so2_rotations(2, 7, 1, buf, buf, None) == 1        # unknown dtype
    assert lib.tpconv_so2_rotations(2, 0, -1, buf, buf, None) == 1
    assert lib.tpconv_so2_rotations(2, 0, 0, None, None, None) == 0       # nothing to do
    assert lib.tpconv_so2_forward(None, 2, 16, 0, None, None, None, None, None) == 1
    assert lib.tpconv_so2_backward(None, 2, 16, 0, *([None] * 7), 0, None) == 1
    assert lib.tpconv_so2_backward_noalloc(None, 2, 16, 0, *([None] * 7)) == 1
    assert lib.tpconv_so2_double_backward(None, 2, 16, 0, *([None] * 10), 0, None) == 1
    assert lib.tpconv_so2_frames_backward(None, 2, 16, 0, *([None] * 6), 0, None) == 1
    assert lib.tpconv_so2_rotations_backward(5, 0, 1, buf, buf, buf, None) == 3
    assert lib.tpconv_so2_rotations_backward(2, 0, 1, None, None, None, None) == 1
    # unsupported shapes and dtypes are refused before the graph is read
    fake = ctypes.c_void_p(ctypes.addressof(buf))
    assert lib.tpconv_so2_forward(fake, 4, 16, 0, None, None, None, None, None) == 3
    assert lib.tpconv_so2_forward(fake, 2, 16, 1, None, None, None, None, None) == 3
    assert lib.tpconv_so2_backward(fake, 2, 64, 0, *([None] * 7), 0, None) == 3
    assert lib.tpconv_so2_backward_noalloc(fake, 2, 64, 0, *([None] * 7)) == 3
    assert lib.tpconv_so2_backward_noalloc(fake, 2, 16, 1, *([None] * 7)) == 3


def test_radial_refusals_need_no_gpu(tp):
    # a zeroed graph struct: no nodes, no edges (nothing is launched)
    lib = tp._lib
    buf = (ctypes.c_uint8 * 256)()
    g = ctypes.c_void_p(ctypes.addressof(buf))
    f32 = tp.tpconv_plan("16x0e+16x1o", 1, "16x0e+16x1o", "f32")
    f64 = tp.tpconv_plan("16x0e+16x1o", 1, "16x0e+16x1o", "f64")
    odd = tp.tpconv_plan("8x0e+8x1o", 1, "8x0e+8x1o", "f32")
    assert lib.tpconv_radial_forward(None, g, 16, *([None] * 5), None) == 1
    assert lib.tpconv_radial_forward(f32.handle, g, 16, *([None] * 5), None) == 0       # nothing to do
    assert lib.tpconv_radial_forward(f64.handle, g, 16, *([None] * 5), None) == 3
    assert lib.tpconv_radial_forward(odd.handle, g, 16, *([None] * 5), None) == 3       # U = 8
    for H in (8, 24, 48, 256):
        assert lib.tpconv_radial_forward(f32.handle, g, H, *([None] * 5), None) == 3
        assert lib.tpconv_radial_backward(f32.handle, g, H, *([None] * 9), None) == 3
    assert lib.tpconv_radial_backward(f32.handle, g, 64, *([None] * 9), None) == 0
    assert "hidden" in tp.tpconv_last_error() or tp.tpconv_last_error()

