"""bench.py's command line on the CPU: the one-GPU contract (no GPU needed)."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes_of_the_4096_atom_workload():
    sys.path.insert(0, ROOT)
    import bench

    class P:  # the plan sizes of 32x0e+32x1o+32x2e+32x3o, SH l<=3 (23 paths)
        weight_numel, dim_sh, dim_in, dim_out = 23 * 32, 16, 512, 512

    fwd, bwd = bench.algorithmic_bytes(P, 4096, 214648, 4)
    assert fwd == 214648 * 3012 + 4096 * (1024 * 4 + 4)
    assert bwd == 214648 * 6024 + 4096 * (1536 * 4 + 4)
    ddf, ddb = bench.dd_algorithmic_bytes(P, 4096, 214648, 4)
    assert ddf == 214648 * ((2 * 736 + 32) * 4 + 4) + 4096 * (1536 * 4 + 4)
    assert ddb == 214648 * ((3 * 736 + 48) * 4 + 8) + 4096 * (2048 * 4 + 4)


def test_kernel_source_hash_ignores_comments():
    """The counters' key covers the compiled code only: comments, trailing
    blanks and blank lines do not change it; a code change does."""
    sys.path.insert(0, ROOT)
    import bench
    code = "int f(int a) {\n  return a + 1;\n}\n"
    annotated = "// adds one\nint f(int a) {  /* the\n argument */\n\n  return a + 1;   // here\n}\n"
    assert bench.strip_comments(code) == bench.strip_comments(annotated)
    assert bench.strip_comments(code) != bench.strip_comments(code.replace("+ 1", "+ 2"))
    h = bench.kernel_source_hash()
    assert len(h) == 16 and h == bench.kernel_source_hash()
