"""Build libtpconv.so (gfx950) in-tree with hipcc.

    python -m equivariant_mlip_tensor_amd.build     # or __graft_entry__.build()

Objects go to <repo>/_build/, the shared library to this package directory.
The kernel translation unit is compiled once per (l bound, data type, kernel
family: forward/backward or double backward) so the twenty objects build in
parallel.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtpconv.so")

ARCH = "gfx950"
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

COMMON = [
    "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
    # packed FP32 (v_pk_*_f32) stays off: plain fp32 FMAs only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero",
    "-fconstexpr-steps=100000000",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _jobs():
    units = []
    for L in (4, 3, 2, 1, 0):          # longest compiles first
        for dd in (1, 0):
            for dbl in (1, 0):
                stem = "tp_dd" if dd else "tp"
                units.append((os.path.join(CSRC, "tp_kernels.hip"),
                              os.path.join(BUILD, f"{stem}_l{L}_{'f64' if dbl else 'f32'}.o"),
                              [f"-DTPCONV_L={L}", f"-DTPCONV_DOUBLE={dbl}", f"-DTPCONV_DD={dd}"]))
    units.append((os.path.join(CSRC, "graph.hip"), os.path.join(BUILD, "graph.o"), []))
    units.append((os.path.join(CSRC, "sh.hip"), os.path.join(BUILD, "sh.o"), []))
    units.append((os.path.join(CSRC, "so2.hip"), os.path.join(BUILD, "so2.o"), []))
    # the host CG builder runs without FMA contraction so its run-time values
    # are bit-identical to the kernels' compile-time evaluation
    units.append((os.path.join(CSRC, "plan.cpp"), os.path.join(BUILD, "plan.o"), ["-ffp-contract=off"]))
    units.append((os.path.join(CSRC, "api.cpp"), os.path.join(BUILD, "api.o"), []))
    return units


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}")
    return r.stdout


def build(verbose: bool = False) -> str:
    """Compile every source and link libtpconv.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = _jobs()

    def compile_one(job):
        src, obj, extra = job
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [HIPCC] + COMMON + extra + lang + ["-c", src, "-o", obj]
        out = _run(cmd)
        if verbose:
            print(" ".join(cmd), flush=True)
        return out

    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(compile_one, jobs))
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + [j[1] for j in jobs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
