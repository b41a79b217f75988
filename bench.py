#!/usr/bin/env python3
"""Forward+backward CGTP convolution throughput on one MI355X.

One step = tpconv_forward + tpconv_backward (dx, dY, dW) over the 4096-atom
SevenNet-l3i5-shaped workload: density 0.1/A^3, periodic box, cutoff 5 A
(~214.6k edges), irreps 32x0e+32x1o+32x2e+32x3o in and out, SH l<=3, all 23
parity-allowed paths, fp32, seeded synthetic inputs resident in HBM.

Prints one JSON line: edges/s (value), per-kernel times, the dominant
kernel's roofline point, and the fp64 CPU oracle timed on a bounded sample
of the same workload.  Outside the timed steps it also reports cold-cache
kernel times (1 GiB read before each step), the double backward's two
kernels (tpconv_double_backward with seeded cotangents), the upstream
kernels (edge harmonics, their gradient, the position gradient; and the
convolution with the harmonics inside its kernels against that three-kernel
chain) and the SO(2)
convolution on the same graph (its rotations, forward, grad_x,
map-gradient, double-backward and frame-gradient passes, against the fp32
matrix-core peak).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
FP32_VALU_PEAK_TFLOPS = 157.3  # 256 CU x 2.4 GHz x 64 lanes x 2 flop x 2 (packed FMA)
FP32_VALU_PLAIN_TFLOPS = 78.6  # the same without packed FMA, which this build does not emit
FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix-core peak


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="c4k")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-edges", type=int, default=40000)
    p.add_argument("--cold-reps", type=int, default=20,
                   help="after the timed steps, this many extra steps each preceded by reading a 1 GiB buffer "
                        "(evicts the 256 MB Infinity Cache); kernel medians reported as kernels_ms_cold")
    p.add_argument("--dd-reps", type=int, default=20,
                   help="timed double-backward calls after the fwd+bwd steps (0 skips); reported as double_backward")
    p.add_argument("--upstream-reps", type=int, default=20,
                   help="timed calls of the edge-harmonics / position-gradient kernels (0 skips); reported as upstream")
    p.add_argument("--so2-reps", type=int, default=20,
                   help="timed calls of each SO(2)-convolution pass on the same graph (0 skips); reported as so2")
    p.add_argument("--radial-reps", type=int, default=20,
                   help="timed calls of the convolution with weights from the radial network's last layer, "
                        "fused and unfused (0 skips); reported as radial")
    p.add_argument("--radial-hidden", type=int, default=64)
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="also run one plain device copy of this many MiB, then a random-order gather of 64-byte "
                        "rows of the same size (scale rocprofv3 FETCH/WRITE_SIZE)")
    return p.parse_args()


def algorithmic_bytes(plan, n_nodes, n_edges, b):
    """Compulsory HBM bytes: every per-edge input read once, every output written once, node rows once."""
    PU, Dsh = plan.weight_numel, plan.dim_sh
    fwd = n_edges * ((PU + Dsh) * b + 4) + n_nodes * ((plan.dim_in + plan.dim_out) * b + 4)
    bwd = n_edges * ((2 * PU + 2 * Dsh) * b + 8) + n_nodes * ((2 * plan.dim_in + plan.dim_out) * b + 4)
    return fwd, bwd


def dd_algorithmic_bytes(plan, n_nodes, n_edges, b):
    """Double backward, compulsory bytes of its two kernels: grad_G pass (reads W, ggW,
    Y, ggY per edge; x, ggx per node; writes grad_G) and the grad_x / grad_Y / grad_W
    pass (reads W, ggW, Y, ggY and writes grad_W, grad_Y per edge; reads x, ggx, G and
    writes grad_x per node)."""
    PU, Dsh, Din, Dout = plan.weight_numel, plan.dim_sh, plan.dim_in, plan.dim_out
    ddf = n_edges * ((2 * PU + 2 * Dsh) * b + 4) + n_nodes * ((2 * Din + Dout) * b + 4)
    ddb = n_edges * ((3 * PU + 3 * Dsh) * b + 8) + n_nodes * ((3 * Din + Dout) * b + 4)
    return ddf, ddb


def so2_flops_per_edge(lmax, C):
    """Dense-map flops per edge: 2 K_0^2 + 4 x 2 K_m^2 for m >= 1 (four K_m x K_m
    products per (+m, -m) pair); the rotations' VALU work is not counted."""
    ks = [(lmax + 1 - m) * C for m in range(lmax + 1)]
    return 2 * (ks[0] ** 2 + 4 * sum(k * k for k in ks[1:]))


def strip_comments(text):
    """C++ source without its comments, trailing blanks and blank lines."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", ln).rstrip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln)


def kernel_source_hash():
    """Hash of the kernel sources' code (comments removed: the counters depend
    on what is compiled, not on how it is annotated)."""
    h = hashlib.sha256()
    for f in ("tp_kernels.hip", "cg_real.hpp", "tp_common.hpp", "sh_eval.hpp"):
        with open(os.path.join(ROOT, "equivariant_mlip_tensor_amd", "csrc", f)) as fh:
            h.update(strip_comments(fh.read()).encode())
    return h.hexdigest()[:16]


def counter_traffic(workload, kernel):
    """Calibrated HBM bytes per launch from the committed rocprofv3 counters,
    or None when they are missing or were taken on another kernel source."""
    path = os.path.join(ROOT, "profiles", f"tpconv_{workload}_counters.json")
    try:
        with open(path) as fh:
            c = json.load(fh)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source") != kernel_source_hash():
        return None
    key = "bwd_kernel" if kernel == "tpconv_backward" else "fwd_kernel"
    v = c.get("hbm_bytes_per_launch", {}).get(key)
    return None if v is None else int(round(v))


def cpu_baseline(w, d, sample_edges):
    """The fp64 numpy oracle, as it stands, on the edges of the first destination rows."""
    import numpy as np
    from oracle import TPProblem, tp_backward, tp_forward
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    prob = TPProblem.build(w.irreps_in, w.sh_lmax, w.irreps_out)
    dst = d["dst"]
    E = len(dst)
    m = min(sample_edges, E)
    # whole destination rows: cut at a row boundary
    last = dst[m - 1]
    m = int(np.searchsorted(dst, last, side="right"))
    sl = slice(0, m)
    t0 = time.perf_counter()
    tp_forward(prob, d["x"], d["Y"][sl], d["W"][sl], d["src"][sl], dst[sl], d["n_nodes"])
    tp_backward(prob, d["x"], d["Y"][sl], d["W"][sl], d["G"], d["src"][sl], dst[sl], d["n_nodes"])
    dt = time.perf_counter() - t0
    return {"value": m / dt, "unit": "edges/s", "cores": int(blas), "kind": "oracle",
            "sample": f"fwd+bwd over the {m} in-edges of destination rows 0..{int(last)} of {E} edges "
                      f"({dt:.1f} s; numpy/BLAS threads {blas}, "
                      f"{len(os.sched_getaffinity(0))} cores available)"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build runs the convolution on a single MI355X; "
              "--gpus above 1 is not supported", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads
    from equivariant_mlip_tensor_amd import tpconv as tp

    w = workloads.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    plan = tp.tpconv_plan(w.irreps_in, w.sh_lmax, w.irreps_out, w.dtype)
    d = workloads.make_inputs(w, plan.n_paths, plan.weight_numel)
    N, E = d["n_nodes"], len(d["src"])
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    src, dst = T(d["src"]), T(d["dst"])
    x, Y, W, G = T(d["x"]), T(d["Y"]), T(d["W"]), T(d["G"])
    t0 = time.perf_counter()
    graph = tp.tpconv_graph_create(N, src, dst)
    torch.cuda.synchronize()
    graph_ms = (time.perf_counter() - t0) * 1e3
    # a rebuild (what a changed neighbour list costs), into the same workspace
    t0 = time.perf_counter()
    graph = tp.tpconv_graph_create(N, src, dst, workspace=graph.workspace)
    torch.cuda.synchronize()
    graph_rebuild_ms = (time.perf_counter() - t0) * 1e3
    out = torch.empty((N, plan.dim_out), dtype=plan.torch_dtype, device=dev)
    dx = torch.empty((N, plan.dim_in), dtype=plan.torch_dtype, device=dev)
    dY = torch.empty((E, plan.dim_sh), dtype=plan.torch_dtype, device=dev)
    dW = torch.empty((E, plan.weight_numel), dtype=plan.torch_dtype, device=dev)

    def step():
        tp.tpconv_forward(plan, graph, x, Y, W, out)
        tp.tpconv_backward(plan, graph, x, Y, W, G, dx, dY, dW)

    # achievable bandwidth on this machine: a 1 GiB device-to-device copy (read +
    # write counted), timed with events, median of 10
    c_src = torch.ones(2**28, dtype=torch.float32, device=dev)
    c_dst = torch.empty_like(c_src)
    c_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(12)]
    for k in range(12):
        c_ev[k][0].record()
        c_dst.copy_(c_src)
        c_ev[k][1].record()
    torch.cuda.synchronize()
    copy_ms = float(np.median([e[0].elapsed_time(e[1]) for e in c_ev[2:]]))
    copy_gbs = 2 * c_src.numel() * 4 / (copy_ms * 1e-3) / 1e9
    del c_src, c_dst
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats()   # the peak reported is the convolution's own

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * 2**20 // 4
        a_src = torch.ones(n, dtype=torch.float32, device=dev)
        a_dst = torch.empty_like(a_src)
        a_dst.copy_(a_src)
        torch.cuda.synchronize()
        # and a gather of the same bytes in random order: rows of 16 floats
        # (64 B) read once each through a random permutation (int64 indices),
        # the access pattern of the kernels' neighbour gathers
        rows = n // 16
        perm = torch.randperm(rows, device=dev)
        torch.cuda.synchronize()
        torch.index_select(a_src.view(rows, 16), 0, perm, out=a_dst.view(rows, 16))
        torch.cuda.synchronize()
        del a_src, a_dst, perm

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()   # the kernels are launched on this stream
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        ev[k][0].record(stream)
        tp.tpconv_forward(plan, graph, x, Y, W, out)
        ev[k][1].record(stream)
        tp.tpconv_backward(plan, graph, x, Y, W, G, dx, dY, dW)
        ev[k][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    bwd_ms = np.array([e[1].elapsed_time(e[2]) for e in ev])
    peak_gib = torch.cuda.max_memory_allocated() / 2**30

    cold = None
    if args.cold_reps > 0:
        # cold-cache kernel times: a 1 GiB read before each step pushes the
        # inputs out of L2 and the Infinity Cache without leaving dirty lines
        evict = torch.ones(2**28, dtype=torch.float32, device=dev)
        cev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.cold_reps)]
        for k in range(args.cold_reps):
            evict.sum()
            cev[k][0].record(stream)
            tp.tpconv_forward(plan, graph, x, Y, W, out)
            cev[k][1].record(stream)
            tp.tpconv_backward(plan, graph, x, Y, W, G, dx, dY, dW)
            cev[k][2].record(stream)
        torch.cuda.synchronize()
        cf = float(np.median([e[0].elapsed_time(e[1]) for e in cev]))
        cb = float(np.median([e[1].elapsed_time(e[2]) for e in cev]))
        cold = {"forward_median": round(cf, 4), "backward_median": round(cb, 4), "reps": args.cold_reps,
                "edges_per_s": round(E / ((cf + cb) * 1e-3), 1),
                "evict": "1 GiB device read (torch.sum) before each step"}
        del evict

    up = None
    if args.upstream_reps > 0:
        # the step upstream of the convolution on the same graph: Y from the
        # edge vectors, grad_vec from dY, grad_pos from grad_vec
        b_ = 4 if w.dtype == "f32" else 8
        vec_t = T(d["vec"].astype(w.np_dtype))
        Y_t = torch.empty_like(Y)
        gv_t = torch.empty_like(vec_t)
        gp_t = torch.empty((N, 3), dtype=plan.torch_dtype, device=dev)
        uev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.upstream_reps + 2)]
        for k in range(args.upstream_reps + 2):   # the first two are warm-up
            uev[k][0].record(stream)
            tp.tpconv_sh(plan, vec_t, Y_t)
            uev[k][1].record(stream)
            tp.tpconv_sh_backward(plan, vec_t, dY, gv_t)
            uev[k][2].record(stream)
            tp.tpconv_positions_backward(plan, graph, gv_t, gp_t)
            uev[k][3].record(stream)
        torch.cuda.synchronize()
        med = [float(np.median([e[i].elapsed_time(e[i + 1]) for e in uev[2:]])) for i in range(3)]
        Dsh = plan.dim_sh
        ub = [E * (3 + Dsh) * b_, E * (6 + Dsh) * b_, E * (3 * b_ + 8) + N * (3 * b_ + 8)]
        up = {name: {"ms_median": round(m, 4), "algorithmic_bytes": int(bb),
                     "algorithmic_GBps": round(bb / (m * 1e-3) / 1e9, 1)}
              for name, m, bb in zip(("tpconv_sh", "tpconv_sh_backward", "tpconv_positions_backward"), med, ub)}
        up["reps"] = args.upstream_reps
        # the force chain's convolution with the harmonics inside its kernels
        # (tpconv_forward_vec, tpconv_backward_vec) against the three-kernel
        # chain around tpconv_forward / tpconv_backward, interleaved
        fev = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.upstream_reps + 2)]
        for k in range(args.upstream_reps + 2):   # the first two are warm-up
            e_ = fev[k]
            e_[0].record(stream)
            tp.tpconv_sh(plan, vec_t, Y_t)
            e_[1].record(stream)
            tp.tpconv_forward(plan, graph, x, Y_t, W, out)
            e_[2].record(stream)
            tp.tpconv_backward(plan, graph, x, Y_t, W, G, dx, dY, dW)
            e_[3].record(stream)
            tp.tpconv_sh_backward(plan, vec_t, dY, gv_t)
            e_[4].record(stream)
            tp.tpconv_forward_vec(plan, graph, x, vec_t, W, out)
            e_[5].record(stream)
            tp.tpconv_backward_vec(plan, graph, x, vec_t, W, G, dx, gv_t, dW)
            e_[6].record(stream)
        torch.cuda.synchronize()
        fm = lambda i, j: float(np.median([e_[i].elapsed_time(e_[j]) for e_ in fev[2:]]))  # noqa: E731
        chain_ms, fused_ms = fm(0, 4), fm(4, 6)
        up["harmonics_in_kernels"] = {
            "three_kernel_chain_ms_median": round(chain_ms, 4),
            "fused_ms_median": round(fused_ms, 4),
            "forward_ms_median": round(fm(1, 2), 4), "backward_ms_median": round(fm(2, 3), 4),
            "forward_vec_ms_median": round(fm(4, 5), 4), "backward_vec_ms_median": round(fm(5, 6), 4),
            "chain_edges_per_s": round(E / (chain_ms * 1e-3), 1), "fused_edges_per_s": round(E / (fused_ms * 1e-3), 1),
            "chain": "tpconv_sh + tpconv_forward + tpconv_backward + tpconv_sh_backward",
            "fused": "tpconv_forward_vec + tpconv_backward_vec"}
        del vec_t, Y_t, gv_t, gp_t

    dd = None
    if args.dd_reps > 0:
        # double backward: the grad_G kernel and the grad_x / grad_Y / grad_W
        # kernel timed separately (two calls, each asking for its outputs)
        ct = workloads.make_cotangents(w, E, plan.weight_numel)
        ga, gb, gc = T(ct["ggx"]), T(ct["ggY"]), T(ct["ggW"])
        del ct
        gx_, gY_, gW_ = torch.empty_like(dx), torch.empty_like(dY), torch.empty_like(dW)
        gG_ = torch.empty((N, plan.dim_out), dtype=plan.torch_dtype, device=dev)

        def dd_call(ev0, ev1, ev2):
            ev0.record(stream)
            tp.tpconv_double_backward(plan, graph, x, Y, W, G, ga, gb, gc, grad_G=gG_,
                                      need=(False, False, False, True))
            ev1.record(stream)
            tp.tpconv_double_backward(plan, graph, x, Y, W, G, ga, gb, gc, gx_, gY_, gW_,
                                      need=(True, True, True, False))
            ev2.record(stream)

        dev_ = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.dd_reps + 2)]
        for k in range(args.dd_reps + 2):   # the first two are warm-up
            dd_call(*dev_[k])
        torch.cuda.synchronize()
        f_ms = np.array([e[0].elapsed_time(e[1]) for e in dev_[2:]])
        b_ms = np.array([e[1].elapsed_time(e[2]) for e in dev_[2:]])
        ddf_bytes, ddb_bytes = dd_algorithmic_bytes(plan, N, E, 4 if w.dtype == "f32" else 8)
        tot = float(np.median(f_ms + b_ms))
        dd = {"grad_G_kernel_ms_median": round(float(np.median(f_ms)), 4),
              "grad_xYW_kernel_ms_median": round(float(np.median(b_ms)), 4),
              "total_ms_median": round(tot, 4), "reps": args.dd_reps,
              "edges_per_s": round(E / (tot * 1e-3), 1),
              "algorithmic_bytes": {"grad_G_kernel": int(ddf_bytes), "grad_xYW_kernel": int(ddb_bytes)},
              "algorithmic_GBps": round((ddf_bytes + ddb_bytes) / (tot * 1e-3) / 1e9, 1),
              "frac_of_peak": round((ddf_bytes + ddb_bytes) / (tot * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del ga, gb, gc, gx_, gY_, gW_, gG_

    so2 = None
    if args.so2_reps > 0 and w.name in workloads.SO2_SHAPES:
        # the SO(2) convolution on the same graph, each pass timed alone
        L2, C2 = workloads.SO2_SHAPES[w.name]
        s2 = workloads.make_so2_inputs(w, tp.tpconv_so2_weight_numel(L2, C2))
        vec2, x2, w2, G2 = T(s2["vec"].astype(np.float32)), T(s2["x"]), T(s2["weights"]), T(s2["G"])
        del s2
        D2 = tp.tpconv_so2_rotations(L2, vec2)
        o2, gx2 = torch.empty_like(x2), torch.empty_like(x2)
        gw2 = torch.empty_like(w2)
        ws2 = torch.empty(tp.tpconv_so2_workspace_bytes(L2, C2, E), dtype=torch.uint8, device=dev)
        ggx2 = torch.randn(x2.shape, dtype=torch.float32, device=dev, generator=torch.Generator(device=dev).manual_seed(5))
        ggw2 = torch.randn(w2.shape, dtype=torch.float32, device=dev, generator=torch.Generator(device=dev).manual_seed(6))
        dd2 = [torch.empty_like(x2), torch.empty_like(w2), torch.empty_like(x2)]
        gD2 = torch.empty_like(D2)
        gv2 = torch.empty_like(vec2)
        dvec2 = torch.randn(vec2.shape, dtype=torch.float32, device=dev,
                            generator=torch.Generator(device=dev).manual_seed(7))
        dD2 = torch.empty_like(D2)
        fdd2 = [torch.empty_like(x2), torch.empty_like(w2), torch.empty_like(x2)]
        wsf2 = torch.empty(tp.tpconv_so2_frames_double_backward_workspace_bytes(L2, C2, N, E), dtype=torch.uint8,
                           device=dev)
        sev = [[torch.cuda.Event(enable_timing=True) for _ in range(10)] for _ in range(args.so2_reps + 2)]
        for k in range(args.so2_reps + 2):   # the first two are warm-up
            sev[k][0].record(stream)
            tp.tpconv_so2_rotations(L2, vec2, D2)
            sev[k][1].record(stream)
            tp.tpconv_so2_forward(graph, L2, C2, x2, D2, w2, o2)
            sev[k][2].record(stream)
            tp.tpconv_so2_backward(graph, L2, C2, x2, D2, w2, G2, grad_x=gx2, need=(True, False))
            sev[k][3].record(stream)
            tp.tpconv_so2_backward(graph, L2, C2, x2, D2, w2, G2, grad_weights=gw2, workspace=ws2,
                                   need=(False, True))
            sev[k][4].record(stream)
            tp.tpconv_so2_double_backward(graph, L2, C2, x2, D2, w2, G2, ggx2, ggw2, *dd2, workspace=ws2)
            sev[k][5].record(stream)
            tp.tpconv_so2_frames_backward(graph, L2, C2, x2, D2, w2, G2, gD2, workspace=ws2)
            sev[k][6].record(stream)
            tp.tpconv_so2_rotations_backward(L2, vec2, gD2, gv2)
            sev[k][7].record(stream)
            tp.tpconv_so2_rotations_jvp(L2, vec2, dvec2, dD2)
            sev[k][8].record(stream)
            tp.tpconv_so2_frames_double_backward(graph, L2, C2, x2, D2, w2, G2, dD2, *fdd2, workspace=wsf2)
            sev[k][9].record(stream)
        torch.cuda.synchronize()
        med = [float(np.median([e[i].elapsed_time(e[i + 1]) for e in sev[2:]])) for i in range(9)]
        fl = so2_flops_per_edge(L2, C2) * E
        tf = lambda ms: round(fl / (ms * 1e-3) / 1e12, 2)   # noqa: E731
        so2 = {"shape": f"l<={L2}, {C2} channels, {N} nodes, {E} edges, fp32",
               "flops_per_pass": int(fl),
               "rotations_ms_median": round(med[0], 4),
               "forward_ms_median": round(med[1], 4), "forward_TFLOPs": tf(med[1]),
               "grad_x_ms_median": round(med[2], 4), "grad_x_TFLOPs": tf(med[2]),
               "grad_weights_ms_median": round(med[3], 4), "grad_weights_TFLOPs": tf(med[3]),
               "roofline": {"bound": "mfma", "kernel": "k_so2_conv (forward)", "achieved": tf(med[1]),
                            "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                            "frac": round(fl / (med[1] * 1e-3) / 1e12 / FP32_MFMA_PEAK_TFLOPS, 4)},
               "fwd_bwd_edges_per_s": round(E / ((med[1] + med[2] + med[3]) * 1e-3), 1),
               "double_backward_ms_median": round(med[4], 4),
               "double_backward_TFLOPs": round(4 * fl / (med[4] * 1e-3) / 1e12, 2),
               "frames_backward_ms_median": round(med[5], 4),
               "rotations_backward_ms_median": round(med[6], 4),
               "rotations_jvp_ms_median": round(med[7], 4),
               "frames_double_backward_ms_median": round(med[8], 4),
               "frames_double_backward_TFLOPs": round(6 * fl / (med[8] * 1e-3) / 1e12, 2),
               "reps": args.so2_reps}
        del vec2, x2, w2, G2, D2, o2, gx2, gw2, ws2, ggx2, ggw2, dd2, gD2, gv2, dvec2, dD2, fdd2, wsf2

    radial = None
    if args.radial_reps > 0 and w.dtype == "f32":
        # W = h M from the radial network's last layer: generated inside the
        # kernels (fused) against the chain that materialises W (a GEMM, the
        # convolution, and the GEMMs for the gradients of h and M)
        H = args.radial_hidden
        gr = torch.Generator(device=dev).manual_seed(11)
        hh = torch.randn((E, H), dtype=torch.float32, device=dev, generator=gr)
        MM = torch.randn((H, plan.weight_numel), dtype=torch.float32, device=dev,
                         generator=gr) / float(np.sqrt(H * plan.n_paths))
        r_out, r_dx, r_dY = torch.empty_like(out), torch.empty_like(dx), torch.empty_like(dY)
        r_dh, r_dW, r_dM = torch.empty_like(hh), torch.empty_like(dW), torch.empty_like(MM)
        Wu = torch.empty_like(dW)
        nev = 11
        rev = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.radial_reps + 2)]
        for k in range(args.radial_reps + 2):   # the first two are warm-up
            ev = rev[k]
            ev[0].record(stream)
            tp.tpconv_radial_forward(plan, graph, x, Y, hh, MM, r_out)
            ev[1].record(stream)
            tp.tpconv_radial_backward(plan, graph, x, Y, hh, MM, G, r_dx, r_dY, r_dh, need=(True, True, True, False))
            ev[2].record(stream)
            tp.tpconv_radial_backward(plan, graph, x, Y, hh, MM, G, r_dx, r_dY, r_dh, r_dW)
            ev[3].record(stream)
            torch.matmul(hh.t(), r_dW, out=r_dM)
            ev[4].record(stream)
            torch.matmul(hh, MM, out=Wu)
            ev[5].record(stream)
            tp.tpconv_forward(plan, graph, x, Y, Wu, out)
            ev[6].record(stream)
            tp.tpconv_backward(plan, graph, x, Y, Wu, G, dx, dY, dW)
            ev[7].record(stream)
            torch.matmul(dW, MM.t(), out=r_dh)
            ev[8].record(stream)
            torch.matmul(hh.t(), dW, out=r_dM)
            ev[9].record(stream)
        torch.cuda.synchronize()
        rm = [float(np.median([e[i].elapsed_time(e[i + 1]) for e in rev[2:]])) for i in range(9)]
        fused_inf = rm[0] + rm[1]
        unfused_inf = rm[4] + rm[5] + rm[6] + rm[7]
        fused_train = rm[0] + rm[2] + rm[3]
        unfused_train = unfused_inf + rm[8]
        gemm_flops = 2.0 * E * H * plan.weight_numel
        radial = {"hidden": H, "weight_columns": plan.weight_numel, "reps": args.radial_reps,
                  "fused": {"forward_ms": round(rm[0], 4), "backward_x_Y_h_ms": round(rm[1], 4),
                            "backward_x_Y_h_W_ms": round(rm[2], 4), "grad_M_gemm_ms": round(rm[3], 4)},
                  "unfused": {"W_gemm_ms": round(rm[4], 4), "forward_ms": round(rm[5], 4),
                              "backward_ms": round(rm[6], 4), "grad_h_gemm_ms": round(rm[7], 4),
                              "grad_M_gemm_ms": round(rm[8], 4)},
                  "inference_ms": {"fused": round(fused_inf, 4), "unfused": round(unfused_inf, 4),
                                   "speedup": round(unfused_inf / fused_inf, 3)},
                  "training_ms": {"fused": round(fused_train, 4), "unfused": round(unfused_train, 4),
                                  "speedup": round(unfused_train / fused_train, 3)},
                  "fused_forward_W_TFLOPs": round(gemm_flops / (rm[0] * 1e-3) / 1e12, 2),
                  "W_bytes_not_moved": int(E * plan.weight_numel * 4)}
        del hh, MM, r_out, r_dx, r_dY, r_dh, r_dW, r_dM, Wu

    b = 4 if w.dtype == "f32" else 8
    fwd_bytes, bwd_bytes = algorithmic_bytes(plan, N, E, b)
    f_avg, b_avg = float(fwd_ms.mean()), float(bwd_ms.mean())
    ms_per_step = wall * 1e3 / args.steps
    dom = ("tpconv_backward", bwd_bytes, b_avg) if b_avg >= f_avg else ("tpconv_forward", fwd_bytes, f_avg)
    achieved = dom[1] / (dom[2] * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": counter_traffic(w.name, dom[0]),
                "kernel": dom[0], "algorithmic_bytes": int(dom[1]), "avg_ms": round(dom[2], 4)}
    hbm_fwdbwd = (fwd_bytes + bwd_bytes) / ((f_avg + b_avg) * 1e-3) / 1e9

    res = {
        "metric": "edges/sec fwd+bwd CGTP conv (l_max=3, 4096 atoms); achieved HBM GB/s % peak",
        "value": round(E * args.steps / wall, 1),
        "unit": "edges/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"{w.name}: {N} atoms, density 0.1/A^3, periodic, cutoff {w.cutoff} A, "
                               f"{E} edges, {w.irreps_in} -> {w.irreps_out}, SH l<={w.sh_lmax}, "
                               f"{plan.n_paths} paths", "n_nodes": N, "n_edges": E},
        "kernels_ms": {"forward_avg": round(f_avg, 4), "forward_median": round(float(np.median(fwd_ms)), 4),
                       "forward_min": round(float(fwd_ms.min()), 4),
                       "backward_avg": round(b_avg, 4), "backward_median": round(float(np.median(bwd_ms)), 4),
                       "backward_min": round(float(bwd_ms.min()), 4)},
        "kernels_ms_cold": cold,
        "double_backward": dd,
        "upstream": up,
        "so2": so2,
        "radial": radial,
        "hbm": {"fwd_bwd_algorithmic_GBps": round(hbm_fwdbwd, 1), "frac_of_peak": round(hbm_fwdbwd / HBM_PEAK_GBS, 4),
                "fwd_bytes": int(fwd_bytes), "bwd_bytes": int(bwd_bytes),
                "copy_1GiB_GBps": round(copy_gbs, 1), "frac_of_copy": round(hbm_fwdbwd / copy_gbs, 4)},
        "roofline": roofline,
        "graph_build_ms": round(graph_ms, 3),
        "graph_rebuild_ms": round(graph_rebuild_ms, 3),
        "peak_device_GiB": round(peak_gib, 3),
        "kernel_source": kernel_source_hash(),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, d, args.cpu_sample_edges)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
