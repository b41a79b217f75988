"""Plain fp64 CPU oracle for the Clebsch-Gordan tensor-product (CGTP) convolution.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code,
tables or constant generators with the HIP library; the only thing both sides
consume is the seeded input generator in ``workloads/``, which holds none of
the method's arithmetic.

What it computes (the LunaTP abstract names the operation "Clebsch--Gordan
tensor product (CGTP) convolution"; the FlashTP summary, sections "Problem" and
"Approach", describes it as a tensor-product layer followed by a reduce layer
over a sparse CG coefficient matrix).  The pages print no formula, so the
plainest reading is used and written out here:

    out[i,s3,u,m3] = sum_{e: dst(e)=i} sum_{p=(s1,l2,s3)} W[e,p,u]
                     sum_{m1,m2} C_p[m1,m2,m3] x[src(e),s1,u,m1] Y[e,l2,m2]

with channelwise ("uvu") coupling, one weight per (edge, path, channel), and
paths into the same output irrep summed with coefficient 1.  Backward gives the
gradients of <G, out> with respect to x, Y and W.

Modules:
  irreps  -- irreps strings and the path list (W layout).
  cg      -- complex CG by Racah's closed form, real-basis CG.
  sh      -- real spherical harmonics built from scipy's complex ones.
  tp      -- dense per-edge forward, backward and double backward.
  forces  -- edge SH with their gradient, and the position gradient.
  so2     -- the SO(2) convolution (edge-frame rotation, per-|m| dense maps,
             inverse rotation on reduction), its backward and double backward,
             and the gradient through the edge frames to the edge vectors.
  radial  -- per-edge weights from the radial network's last layer, W = h M,
             and the convolution's gradients with respect to h and M.

Every function here is pinned by a test in ``tests/test_oracle_*.py`` against
mathematics it does not itself use (library routines, closed forms,
invariants, finite differences, brute force).
"""

from .irreps import Irreps, parse_irreps, enumerate_paths  # noqa: F401
from .cg import cg_complex, real_basis_U, cg_real  # noqa: F401
from .sh import sh_complex, sh_real  # noqa: F401
from .tp import TPProblem, tp_forward, tp_backward, tp_double_backward  # noqa: F401
from .forces import sh_and_jacobian, sh_edges, sh_backward, positions_backward  # noqa: F401
from .radial import radial_weights, radial_forward, radial_backward  # noqa: F401
from .so2 import (edge_rotation, wigner_D, edge_wigner, so2_forward, so2_backward,  # noqa: F401
                  so2_double_backward, so2_frames_backward, rotations_backward,
                  rotations_jvp, so2_frames_double_backward,
                  weight_numel as so2_weight_numel)
