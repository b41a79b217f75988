"""ctypes binding of libtpconv.so: the C entry points under the same names.

Argument marshalling only: torch supplies device memory and the stream, every
step of the convolution runs in the library's HIP kernels.  Importing this
module loads the library and raises if it is missing -- there is no fallback.

    plan  = tpconv_plan("32x0e+32x1o", 1, "32x0e+32x1o", "f32")
    graph = tpconv_graph_create(n_nodes, src, dst)          # src, dst: int32 cuda
    out   = tpconv_forward(plan, graph, x, Y, W)
    dx, dY, dW = tpconv_backward(plan, graph, x, Y, W, grad_out)

The layouts are those of include/tpconv.h.
"""

from __future__ import annotations

import ctypes
import functools
import os
from typing import Optional, Tuple

import torch  # loads the HIP runtime the library then binds to

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtpconv.so")

F32, F64 = 0, 1
STATUS = {0: "TPCONV_OK", 1: "TPCONV_E_INVALID_ARG", 2: "TPCONV_E_IRREPS", 3: "TPCONV_E_UNSUPPORTED",
          4: "TPCONV_E_NO_PATHS", 5: "TPCONV_E_WORKSPACE", 6: "TPCONV_E_INDEX", 7: "TPCONV_E_HIP"}

EXPORTS = ("tpconv_plan", "tpconv_plan_query", "tpconv_plan_paths", "tpconv_plan_table", "tpconv_plan_destroy",
           "tpconv_graph_workspace_bytes", "tpconv_graph_create", "tpconv_graph_export", "tpconv_graph_destroy",
           "tpconv_forward", "tpconv_backward", "tpconv_double_backward", "tpconv_radial_forward",
           "tpconv_radial_backward", "tpconv_sh", "tpconv_sh_backward", "tpconv_forward_vec", "tpconv_backward_vec",
           "tpconv_positions_backward", "tpconv_so2_weight_numel", "tpconv_so2_rotations", "tpconv_so2_forward",
           "tpconv_so2_workspace_bytes", "tpconv_so2_backward", "tpconv_so2_backward_noalloc",
           "tpconv_so2_double_backward",
           "tpconv_so2_frames_backward", "tpconv_so2_rotations_backward", "tpconv_so2_rotations_jvp",
           "tpconv_so2_frames_double_backward_workspace_bytes", "tpconv_so2_frames_double_backward",
           "tpconv_last_error")


class TPConvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.name = STATUS.get(status, str(status))


class PlanInfo(ctypes.Structure):
    _fields_ = [("dim_in", ctypes.c_int64), ("dim_out", ctypes.c_int64), ("dim_sh", ctypes.c_int64),
                ("n_paths", ctypes.c_int64), ("weight_numel", ctypes.c_int64), ("cg_nnz", ctypes.c_int64),
                ("cg_nvalues", ctypes.c_int64), ("mul", ctypes.c_int64), ("kernel_lmax", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run __graft_entry__.build() "
                          "(python -m equivariant_mlip_tensor_amd.build)")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "tpconv_plan": (i32, [ctypes.c_char_p, ctypes.c_int, ctypes.c_char_p, ctypes.c_int, ctypes.POINTER(vp)]),
        "tpconv_plan_query": (i32, [vp, ctypes.POINTER(PlanInfo)]),
        "tpconv_plan_paths": (i32, [vp, vp]),
        "tpconv_plan_table": (i32, [vp, vp, vp, vp]),
        "tpconv_plan_destroy": (None, [vp]),
        "tpconv_graph_workspace_bytes": (sz, [i64, i64]),
        "tpconv_graph_create": (i32, [i64, i64, vp, vp, vp, sz, vp, ctypes.POINTER(vp)]),
        "tpconv_graph_export": (i32, [vp, vp, vp, vp, vp, vp, vp, vp]),
        "tpconv_graph_destroy": (None, [vp]),
        "tpconv_radial_forward": (i32, [vp, vp, i32, vp, vp, vp, vp, vp, vp]),
        "tpconv_radial_backward": (i32, [vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
        "tpconv_forward": (i32, [vp, vp, vp, vp, vp, vp, vp]),
        "tpconv_backward": (i32, [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
        "tpconv_double_backward": (i32, [vp] * 14),
        "tpconv_forward_vec": (i32, [vp, vp, vp, vp, vp, vp, vp]),
        "tpconv_backward_vec": (i32, [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
        "tpconv_sh": (i32, [vp, i64, vp, vp, vp]),
        "tpconv_sh_backward": (i32, [vp, i64, vp, vp, vp, vp]),
        "tpconv_positions_backward": (i32, [vp, vp, vp, vp, vp]),
        "tpconv_so2_weight_numel": (i64, [ctypes.c_int, ctypes.c_int]),
        "tpconv_so2_rotations": (i32, [ctypes.c_int, ctypes.c_int, i64, vp, vp, vp]),
        "tpconv_so2_forward": (i32, [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp]),
        "tpconv_so2_workspace_bytes": (sz, [ctypes.c_int, ctypes.c_int, i64]),
        "tpconv_so2_backward": (i32, [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, sz,
                                      vp]),
        "tpconv_so2_backward_noalloc": (i32, [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int] + [vp] * 7),
        "tpconv_so2_double_backward": (i32, [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int] + [vp] * 10 + [sz, vp]),
        "tpconv_so2_frames_backward": (i32, [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int] + [vp] * 6 + [sz, vp]),
        "tpconv_so2_rotations_backward": (i32, [ctypes.c_int, ctypes.c_int, i64, vp, vp, vp, vp]),
        "tpconv_so2_rotations_jvp": (i32, [ctypes.c_int, ctypes.c_int, i64, vp, vp, vp, vp]),
        "tpconv_so2_frames_double_backward_workspace_bytes": (sz, [ctypes.c_int, ctypes.c_int, i64, i64]),
        "tpconv_so2_frames_double_backward": (i32, [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int] + [vp] * 9 +
                                              [sz, vp]),
        "tpconv_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()


def _check(status: int) -> None:
    if status != 0:
        raise TPConvError(status, _lib.tpconv_last_error().decode(errors="replace"))


def tpconv_last_error() -> str:
    return _lib.tpconv_last_error().decode(errors="replace")


def _stream_handle(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on_launch_stream(fn):
    """Run a wrapper with its launch stream current, so the outputs and
    workspaces it allocates come from that stream's pool: torch's caching
    allocator does not hand such a block to other work before what was queued
    on that stream has passed (a workspace freed when the wrapper returns may
    still be in use by the kernels it launched)."""
    @functools.wraps(fn)
    def wrapper(*args, stream=None, **kw):
        if stream is None:
            return fn(*args, **kw)
        with torch.cuda.stream(stream):
            return fn(*args, stream=stream, **kw)
    return wrapper


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# ---------------------------------------------------------------------- plans
class Plan:
    """Owns a tpconv_plan_t; sizes as attributes."""

    def __init__(self, handle: ctypes.c_void_p):
        self.handle = handle
        info = PlanInfo()
        _check(_lib.tpconv_plan_query(handle, ctypes.byref(info)))
        self.info = info
        for f, _ in PlanInfo._fields_:
            setattr(self, f, getattr(info, f))
        self.torch_dtype = torch.float32 if info.dtype == F32 else torch.float64

    def __del__(self):
        h, self.handle = getattr(self, "handle", None), None
        if h and _lib is not None:
            _lib.tpconv_plan_destroy(h)


def tpconv_plan(irreps_in: str, sh_lmax: int, irreps_out: str, dtype="f32") -> Plan:
    dt = {"f32": F32, "f64": F64, torch.float32: F32, torch.float64: F64, F32: F32, F64: F64}.get(dtype, dtype)
    h = ctypes.c_void_p()
    _check(_lib.tpconv_plan(irreps_in.encode(), int(sh_lmax), irreps_out.encode(), int(dt), ctypes.byref(h)))
    return Plan(h)


def tpconv_plan_query(plan: Plan) -> PlanInfo:
    info = PlanInfo()
    _check(_lib.tpconv_plan_query(plan.handle, ctypes.byref(info)))
    return info


def tpconv_plan_paths(plan: Plan):
    """List of (s1, l2, s3, weight_offset)."""
    buf = (ctypes.c_int32 * (4 * plan.n_paths))()
    _check(_lib.tpconv_plan_paths(plan.handle, buf))
    return [tuple(buf[4 * i:4 * i + 4]) for i in range(plan.n_paths)]


def tpconv_plan_table(plan: Plan):
    """(entries uint32 [nnz], path_ptr int32 [P+1], values float64 [nvalues]) as Python lists."""
    ent = (ctypes.c_uint32 * max(1, plan.cg_nnz))()
    ptr = (ctypes.c_int32 * (plan.n_paths + 1))()
    val = (ctypes.c_double * max(1, plan.cg_nvalues))()
    _check(_lib.tpconv_plan_table(plan.handle, ent, ptr, val))
    return list(ent)[:plan.cg_nnz], list(ptr), list(val)[:plan.cg_nvalues]


def tpconv_plan_destroy(plan: Plan) -> None:
    plan.__del__()


# --------------------------------------------------------------------- graphs
def tpconv_graph_workspace_bytes(n_nodes: int, n_edges: int) -> int:
    return int(_lib.tpconv_graph_workspace_bytes(int(n_nodes), int(n_edges)))


class Graph:
    """Owns a tpconv_graph_t and the device workspace tensor it lives in."""

    def __init__(self, handle, workspace: torch.Tensor, n_nodes: int, n_edges: int):
        self.handle, self.workspace, self.n_nodes, self.n_edges = handle, workspace, n_nodes, n_edges

    def __del__(self):
        h, self.handle = getattr(self, "handle", None), None
        if h and _lib is not None:
            _lib.tpconv_graph_destroy(h)


@_on_launch_stream
def tpconv_graph_create(n_nodes: int, src: torch.Tensor, dst: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                        stream=None) -> Graph:
    if src.dtype != torch.int32 or dst.dtype != torch.int32 or not src.is_cuda or not dst.is_cuda:
        raise TypeError("src and dst must be int32 device tensors")
    if src.shape != dst.shape or src.dim() != 1:
        raise ValueError("src and dst must be 1-D and of equal length")
    src, dst = src.contiguous(), dst.contiguous()
    n_edges = src.numel()
    need = tpconv_graph_workspace_bytes(n_nodes, n_edges)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=src.device)
    h = ctypes.c_void_p()
    _check(_lib.tpconv_graph_create(int(n_nodes), int(n_edges), _ptr(src), _ptr(dst), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream_handle(stream),
                                    ctypes.byref(h)))
    return Graph(h, workspace, int(n_nodes), int(n_edges))


@_on_launch_stream
def tpconv_graph_export(graph: Graph, stream=None):
    """Host copies (numpy int32) of dst_row_ptr, dst_col, dst_eid, src_row_ptr, src_col, src_eid."""
    import numpy as np
    n, e = graph.n_nodes, graph.n_edges
    arrs = [np.zeros(n + 1, np.int32), np.zeros(e, np.int32), np.zeros(e, np.int32),
            np.zeros(n + 1, np.int32), np.zeros(e, np.int32), np.zeros(e, np.int32)]
    _check(_lib.tpconv_graph_export(graph.handle, *[ctypes.c_void_p(a.ctypes.data) for a in arrs],
                                    _stream_handle(stream)))
    return arrs


def tpconv_graph_destroy(graph: Graph) -> None:
    graph.__del__()


# -------------------------------------------------------------------- compute
def _need(t, shape, dtype, name):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda or t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous {dtype} cuda tensor of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)} (cuda={t.is_cuda}, contiguous={t.is_contiguous()})")
    return t


@_on_launch_stream
def tpconv_forward(plan: Plan, graph: Graph, x, Y, W, out=None, stream=None) -> torch.Tensor:
    N, E, dt = graph.n_nodes, graph.n_edges, plan.torch_dtype
    _need(x, (N, plan.dim_in), dt, "x")
    _need(Y, (E, plan.dim_sh), dt, "Y")
    _need(W, (E, plan.weight_numel), dt, "W")
    if out is None:
        out = torch.empty((N, plan.dim_out), dtype=dt, device=x.device)
    _need(out, (N, plan.dim_out), dt, "out")
    _check(_lib.tpconv_forward(plan.handle, graph.handle, _ptr(x), _ptr(Y), _ptr(W), _ptr(out),
                               _stream_handle(stream)))
    return out


@_on_launch_stream
def tpconv_backward(plan: Plan, graph: Graph, x, Y, W, grad_out, grad_x=None, grad_Y=None, grad_W=None,
                    need=(True, True, True), stream=None) -> Tuple[Optional[torch.Tensor], ...]:
    """Returns (grad_x, grad_Y, grad_W); an output is None when `need` turns it off."""
    N, E, dt = graph.n_nodes, graph.n_edges, plan.torch_dtype
    _need(x, (N, plan.dim_in), dt, "x")
    _need(Y, (E, plan.dim_sh), dt, "Y")
    _need(W, (E, plan.weight_numel), dt, "W")
    _need(grad_out, (N, plan.dim_out), dt, "grad_out")
    dev = x.device
    if need[0] and grad_x is None:
        grad_x = torch.empty((N, plan.dim_in), dtype=dt, device=dev)
    if need[1] and grad_Y is None:
        grad_Y = torch.empty((E, plan.dim_sh), dtype=dt, device=dev)
    if need[2] and grad_W is None:
        grad_W = torch.empty((E, plan.weight_numel), dtype=dt, device=dev)
    for t, shp, nm in ((grad_x, (N, plan.dim_in), "grad_x"), (grad_Y, (E, plan.dim_sh), "grad_Y"),
                       (grad_W, (E, plan.weight_numel), "grad_W")):
        if t is not None:
            _need(t, shp, dt, nm)
    _check(_lib.tpconv_backward(plan.handle, graph.handle, _ptr(x), _ptr(Y), _ptr(W), _ptr(grad_out),
                                _ptr(grad_x), _ptr(grad_Y), _ptr(grad_W), _stream_handle(stream)))
    return grad_x, grad_Y, grad_W


@_on_launch_stream
def tpconv_radial_forward(plan: Plan, graph: Graph, x, Y, h, M, out=None, stream=None) -> torch.Tensor:
    """out = tpconv_forward(x, Y, W = h @ M) with W generated inside the kernel.
    h: [E, hidden], M: [hidden, weight_numel], fp32, hidden in 16/32/64/128."""
    N, E, dt = graph.n_nodes, graph.n_edges, plan.torch_dtype
    H = int(M.shape[0])
    _need(x, (N, plan.dim_in), dt, "x")
    _need(Y, (E, plan.dim_sh), dt, "Y")
    _need(h, (E, H), dt, "h")
    _need(M, (H, plan.weight_numel), dt, "M")
    if out is None:
        out = torch.empty((N, plan.dim_out), dtype=dt, device=x.device)
    _need(out, (N, plan.dim_out), dt, "out")
    _check(_lib.tpconv_radial_forward(plan.handle, graph.handle, H, _ptr(x), _ptr(Y), _ptr(h), _ptr(M), _ptr(out),
                                      _stream_handle(stream)))
    return out


@_on_launch_stream
def tpconv_radial_backward(plan: Plan, graph: Graph, x, Y, h, M, grad_out, grad_x=None, grad_Y=None, grad_h=None,
                           grad_W=None, need=(True, True, True, False),
                           stream=None) -> Tuple[Optional[torch.Tensor], ...]:
    """(grad_x, grad_Y, grad_h, grad_W) of <grad_out, tpconv_radial_forward(...)>;
    grad_W (for the caller's grad_M = h^T grad_W) only when need[3]; an output
    is None when `need` turns it off."""
    N, E, dt = graph.n_nodes, graph.n_edges, plan.torch_dtype
    H = int(M.shape[0])
    _need(x, (N, plan.dim_in), dt, "x")
    _need(Y, (E, plan.dim_sh), dt, "Y")
    _need(h, (E, H), dt, "h")
    _need(M, (H, plan.weight_numel), dt, "M")
    _need(grad_out, (N, plan.dim_out), dt, "grad_out")
    dev = x.device
    shapes = ((N, plan.dim_in), (E, plan.dim_sh), (E, H), (E, plan.weight_numel))
    outs = [grad_x, grad_Y, grad_h, grad_W]
    for k, (t, shp, nm) in enumerate(zip(outs, shapes, ("grad_x", "grad_Y", "grad_h", "grad_W"))):
        if need[k] and t is None:
            outs[k] = t = torch.empty(shp, dtype=dt, device=dev)
        if t is not None:
            _need(t, shp, dt, nm)
    _check(_lib.tpconv_radial_backward(plan.handle, graph.handle, H, _ptr(x), _ptr(Y), _ptr(h), _ptr(M),
                                       _ptr(grad_out), *[_ptr(t) for t in outs], _stream_handle(stream)))
    return tuple(outs)


@_on_launch_stream
def tpconv_double_backward(plan: Plan, graph: Graph, x, Y, W, grad_out, ggx=None, ggY=None, ggW=None,
                           grad_x=None, grad_Y=None, grad_W=None, grad_G=None,
                           need=(True, True, True, True), stream=None) -> Tuple[Optional[torch.Tensor], ...]:
    """Gradients of <ggx, dx> + <ggY, dY> + <ggW, dW> (dx, dY, dW = the backward
    of x, Y, W, grad_out) with respect to x, Y, W and grad_out.

    ggx / ggY / ggW may be None (zero).  Returns (grad_x, grad_Y, grad_W,
    grad_G); an output is None when `need` turns it off."""
    N, E, dt = graph.n_nodes, graph.n_edges, plan.torch_dtype
    _need(x, (N, plan.dim_in), dt, "x")
    _need(Y, (E, plan.dim_sh), dt, "Y")
    _need(W, (E, plan.weight_numel), dt, "W")
    if grad_out is not None:
        _need(grad_out, (N, plan.dim_out), dt, "grad_out")
    for t, shp, nm in ((ggx, (N, plan.dim_in), "ggx"), (ggY, (E, plan.dim_sh), "ggY"),
                       (ggW, (E, plan.weight_numel), "ggW")):
        if t is not None:
            _need(t, shp, dt, nm)
    dev = x.device
    shapes = ((N, plan.dim_in), (E, plan.dim_sh), (E, plan.weight_numel), (N, plan.dim_out))
    outs = [grad_x, grad_Y, grad_W, grad_G]
    for k in range(4):
        if need[k] and outs[k] is None:
            outs[k] = torch.empty(shapes[k], dtype=dt, device=dev)
        if outs[k] is not None:
            _need(outs[k], shapes[k], dt, ("grad_x", "grad_Y", "grad_W", "grad_G")[k])
    _check(_lib.tpconv_double_backward(plan.handle, graph.handle, _ptr(x), _ptr(Y), _ptr(W), _ptr(grad_out),
                                       _ptr(ggx), _ptr(ggY), _ptr(ggW), _ptr(outs[0]), _ptr(outs[1]),
                                       _ptr(outs[2]), _ptr(outs[3]), _stream_handle(stream)))
    return tuple(outs)


# ------------------------------------------------- upstream: harmonics, forces
@_on_launch_stream
def tpconv_sh(plan: Plan, vec, Y=None, stream=None) -> torch.Tensor:
    """Y [E, (sh_lmax+1)^2] of the edge vectors vec [E, 3] (plan dtype)."""
    E = vec.shape[0] if vec.dim() == 2 else -1
    _need(vec, (E, 3), plan.torch_dtype, "vec")
    if Y is None:
        Y = torch.empty((E, plan.dim_sh), dtype=plan.torch_dtype, device=vec.device)
    _need(Y, (E, plan.dim_sh), plan.torch_dtype, "Y")
    _check(_lib.tpconv_sh(plan.handle, E, _ptr(vec), _ptr(Y), _stream_handle(stream)))
    return Y


@_on_launch_stream
def tpconv_sh_backward(plan: Plan, vec, grad_Y, grad_vec=None, stream=None) -> torch.Tensor:
    """grad_vec [E, 3] from grad_Y [E, (sh_lmax+1)^2]."""
    E = vec.shape[0] if vec.dim() == 2 else -1
    _need(vec, (E, 3), plan.torch_dtype, "vec")
    _need(grad_Y, (E, plan.dim_sh), plan.torch_dtype, "grad_Y")
    if grad_vec is None:
        grad_vec = torch.empty((E, 3), dtype=plan.torch_dtype, device=vec.device)
    _need(grad_vec, (E, 3), plan.torch_dtype, "grad_vec")
    _check(_lib.tpconv_sh_backward(plan.handle, E, _ptr(vec), _ptr(grad_Y), _ptr(grad_vec), _stream_handle(stream)))
    return grad_vec


@_on_launch_stream
def tpconv_forward_vec(plan: Plan, graph: Graph, x, vec, W, out=None, stream=None) -> torch.Tensor:
    """out = tpconv_forward(x, tpconv_sh(vec), W), the harmonics evaluated inside the kernel."""
    N, E, dt = graph.n_nodes, graph.n_edges, plan.torch_dtype
    _need(x, (N, plan.dim_in), dt, "x")
    _need(vec, (E, 3), dt, "vec")
    _need(W, (E, plan.weight_numel), dt, "W")
    if out is None:
        out = torch.empty((N, plan.dim_out), dtype=dt, device=x.device)
    _need(out, (N, plan.dim_out), dt, "out")
    _check(_lib.tpconv_forward_vec(plan.handle, graph.handle, _ptr(x), _ptr(vec), _ptr(W), _ptr(out),
                                   _stream_handle(stream)))
    return out


@_on_launch_stream
def tpconv_backward_vec(plan: Plan, graph: Graph, x, vec, W, grad_out, grad_x=None, grad_vec=None, grad_W=None,
                        need=(True, True, True), stream=None) -> Tuple[Optional[torch.Tensor], ...]:
    """Returns (grad_x, grad_vec, grad_W) with the harmonics of vec evaluated inside the kernel;
    an output is None when `need` turns it off."""
    N, E, dt = graph.n_nodes, graph.n_edges, plan.torch_dtype
    _need(x, (N, plan.dim_in), dt, "x")
    _need(vec, (E, 3), dt, "vec")
    _need(W, (E, plan.weight_numel), dt, "W")
    _need(grad_out, (N, plan.dim_out), dt, "grad_out")
    dev = x.device
    if need[0] and grad_x is None:
        grad_x = torch.empty((N, plan.dim_in), dtype=dt, device=dev)
    if need[1] and grad_vec is None:
        grad_vec = torch.empty((E, 3), dtype=dt, device=dev)
    if need[2] and grad_W is None:
        grad_W = torch.empty((E, plan.weight_numel), dtype=dt, device=dev)
    for t, shp, nm in ((grad_x, (N, plan.dim_in), "grad_x"), (grad_vec, (E, 3), "grad_vec"),
                       (grad_W, (E, plan.weight_numel), "grad_W")):
        if t is not None:
            _need(t, shp, dt, nm)
    _check(_lib.tpconv_backward_vec(plan.handle, graph.handle, _ptr(x), _ptr(vec), _ptr(W), _ptr(grad_out),
                                    _ptr(grad_x), _ptr(grad_vec), _ptr(grad_W), _stream_handle(stream)))
    return grad_x, grad_vec, grad_W


@_on_launch_stream
def tpconv_positions_backward(plan: Plan, graph: Graph, grad_vec, grad_pos=None, stream=None) -> torch.Tensor:
    """grad_pos [N, 3] for vec[e] = pos[src[e]] - pos[dst[e]] (+ constant shift)."""
    N, E = graph.n_nodes, graph.n_edges
    _need(grad_vec, (E, 3), plan.torch_dtype, "grad_vec")
    if grad_pos is None:
        grad_pos = torch.empty((N, 3), dtype=plan.torch_dtype, device=grad_vec.device)
    _need(grad_pos, (N, 3), plan.torch_dtype, "grad_pos")
    _check(_lib.tpconv_positions_backward(plan.handle, graph.handle, _ptr(grad_vec), _ptr(grad_pos),
                                          _stream_handle(stream)))
    return grad_pos


# ---------------------------------------------------------- SO(2) convolution
def tpconv_so2_weight_numel(lmax: int, channels: int) -> int:
    """Length of the map weights A_0, A_1, B_1, ..., A_L, B_L (0: unsupported)."""
    return int(_lib.tpconv_so2_weight_numel(int(lmax), int(channels)))


def _so2_sizes(lmax, channels):
    nw = tpconv_so2_weight_numel(lmax, channels)
    if nw == 0:
        raise TPConvError(3, f"SO(2) convolution: unsupported lmax={lmax}, channels={channels}")
    return channels * (lmax + 1) ** 2, (lmax + 1) * (2 * lmax + 1) * (2 * lmax + 3) // 3, nw


@_on_launch_stream
def tpconv_so2_rotations(lmax: int, vec, D=None, stream=None) -> torch.Tensor:
    """D [E, sum_l (2l+1)^2]: real Wigner blocks of each edge's frame rotation
    (dtype of vec, float32 or float64)."""
    E = vec.shape[0] if vec.dim() == 2 else -1
    dt = vec.dtype
    _need(vec, (E, 3), dt, "vec")
    nd = (lmax + 1) * (2 * lmax + 1) * (2 * lmax + 3) // 3
    if D is None:
        D = torch.empty((E, nd), dtype=dt, device=vec.device)
    _need(D, (E, nd), dt, "D")
    _check(_lib.tpconv_so2_rotations(int(lmax), F64 if dt == torch.float64 else F32, E, _ptr(vec), _ptr(D),
                                     _stream_handle(stream)))
    return D


@_on_launch_stream
def tpconv_so2_forward(graph: Graph, lmax: int, channels: int, x, D, weights, out=None, stream=None) -> torch.Tensor:
    """out [N, C (L+1)^2] = sum over in-edges of D^T SO2(D x[src])."""
    N, E = graph.n_nodes, graph.n_edges
    dn, nd, nw = _so2_sizes(lmax, channels)
    f = torch.float32
    _need(x, (N, dn), f, "x")
    _need(D, (E, nd), f, "D")
    _need(weights, (nw,), f, "weights")
    if out is None:
        out = torch.empty((N, dn), dtype=f, device=x.device)
    _need(out, (N, dn), f, "out")
    _check(_lib.tpconv_so2_forward(graph.handle, int(lmax), int(channels), F32, _ptr(x), _ptr(D), _ptr(weights),
                                   _ptr(out), _stream_handle(stream)))
    return out


def tpconv_so2_workspace_bytes(lmax: int, channels: int, n_edges: int) -> int:
    return int(_lib.tpconv_so2_workspace_bytes(int(lmax), int(channels), int(n_edges)))


@_on_launch_stream
def tpconv_so2_backward(graph: Graph, lmax: int, channels: int, x, D, weights, grad_out, grad_x=None,
                        grad_weights=None, workspace=None, need=(True, True),
                        stream=None) -> Tuple[Optional[torch.Tensor], Optional[torch.Tensor]]:
    """(grad_x, grad_weights) of <grad_out, out>; an output is None when `need` turns it off."""
    N, E = graph.n_nodes, graph.n_edges
    dn, nd, nw = _so2_sizes(lmax, channels)
    f = torch.float32
    _need(x, (N, dn), f, "x")
    _need(D, (E, nd), f, "D")
    _need(weights, (nw,), f, "weights")
    _need(grad_out, (N, dn), f, "grad_out")
    dev = x.device
    if need[0] and grad_x is None:
        grad_x = torch.empty((N, dn), dtype=f, device=dev)
    if need[1] and grad_weights is None:
        grad_weights = torch.empty((nw,), dtype=f, device=dev)
    if grad_x is not None:
        _need(grad_x, (N, dn), f, "grad_x")
    if grad_weights is not None:
        _need(grad_weights, (nw,), f, "grad_weights")
    ws_bytes = 0
    if grad_x is not None or grad_weights is not None:
        if workspace is None:
            workspace = torch.empty(max(tpconv_so2_workspace_bytes(lmax, channels, E), 256), dtype=torch.uint8,
                                    device=dev)
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.tpconv_so2_backward(graph.handle, int(lmax), int(channels), F32, _ptr(x), _ptr(D), _ptr(weights),
                                    _ptr(grad_out), _ptr(grad_x), _ptr(grad_weights), _ptr(workspace), ws_bytes,
                                    _stream_handle(stream)))
    return grad_x, grad_weights


@_on_launch_stream
def tpconv_so2_backward_noalloc(graph: Graph, lmax: int, channels: int, x, D, weights, grad_out, grad_x,
                                grad_weights, stream=None) -> None:
    """tpconv_so2_backward into caller-given outputs (either may be None), with no
    workspace: the library's device scratch holds the temporaries, so the call
    allocates nothing.  Calls that overlap on one device race on that scratch."""
    N, E = graph.n_nodes, graph.n_edges
    dn, nd, nw = _so2_sizes(lmax, channels)
    f = torch.float32
    _need(x, (N, dn), f, "x")
    _need(D, (E, nd), f, "D")
    _need(weights, (nw,), f, "weights")
    _need(grad_out, (N, dn), f, "grad_out")
    if grad_x is not None:
        _need(grad_x, (N, dn), f, "grad_x")
    if grad_weights is not None:
        _need(grad_weights, (nw,), f, "grad_weights")
    _check(_lib.tpconv_so2_backward_noalloc(graph.handle, int(lmax), int(channels), F32, _ptr(x), _ptr(D),
                                            _ptr(weights), _ptr(grad_out), _ptr(grad_x), _ptr(grad_weights),
                                            _stream_handle(stream)))


@_on_launch_stream
def tpconv_so2_double_backward(graph: Graph, lmax: int, channels: int, x, D, weights, grad_out, ggx=None, ggw=None,
                               grad_x=None, grad_weights=None, grad_G=None, workspace=None,
                               need=(True, True, True), stream=None):
    """Gradients of <ggx, grad_x> + <ggw, grad_w> (the backward's outputs) with
    respect to x, the maps and grad_out; ggx / ggw may be None (zero).
    Returns (grad_x, grad_weights, grad_G); an output is None when `need`
    turns it off."""
    N, E = graph.n_nodes, graph.n_edges
    dn, nd, nw = _so2_sizes(lmax, channels)
    f = torch.float32
    _need(x, (N, dn), f, "x")
    _need(D, (E, nd), f, "D")
    _need(weights, (nw,), f, "weights")
    _need(grad_out, (N, dn), f, "grad_out")
    if ggx is not None:
        _need(ggx, (N, dn), f, "ggx")
    if ggw is not None:
        _need(ggw, (nw,), f, "ggw")
    dev = x.device
    outs = [grad_x, grad_weights, grad_G]
    shapes = ((N, dn), (nw,), (N, dn))
    for k in range(3):
        if need[k] and outs[k] is None:
            outs[k] = torch.empty(shapes[k], dtype=f, device=dev)
        if outs[k] is not None:
            _need(outs[k], shapes[k], f, ("grad_x", "grad_weights", "grad_G")[k])
    ws_bytes = 0
    if outs[0] is not None or outs[1] is not None:
        if workspace is None:
            workspace = torch.empty(max(tpconv_so2_workspace_bytes(lmax, channels, E), 256), dtype=torch.uint8,
                                    device=dev)
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.tpconv_so2_double_backward(graph.handle, int(lmax), int(channels), F32, _ptr(x), _ptr(D),
                                           _ptr(weights), _ptr(grad_out), _ptr(ggx), _ptr(ggw), _ptr(outs[0]),
                                           _ptr(outs[1]), _ptr(outs[2]), _ptr(workspace), ws_bytes,
                                           _stream_handle(stream)))
    return tuple(outs)


@_on_launch_stream
def tpconv_so2_frames_backward(graph: Graph, lmax: int, channels: int, x, D, weights, grad_out, grad_D=None,
                               workspace=None, stream=None) -> torch.Tensor:
    """grad_D [E, sum (2l+1)^2]: gradient of <grad_out, out> with respect to the Wigner blocks."""
    N, E = graph.n_nodes, graph.n_edges
    dn, nd, nw = _so2_sizes(lmax, channels)
    f = torch.float32
    _need(x, (N, dn), f, "x")
    _need(D, (E, nd), f, "D")
    _need(weights, (nw,), f, "weights")
    _need(grad_out, (N, dn), f, "grad_out")
    if grad_D is None:
        grad_D = torch.empty((E, nd), dtype=f, device=x.device)
    _need(grad_D, (E, nd), f, "grad_D")
    if workspace is None:
        workspace = torch.empty(max(tpconv_so2_workspace_bytes(lmax, channels, E), 256), dtype=torch.uint8,
                                device=x.device)
    _check(_lib.tpconv_so2_frames_backward(graph.handle, int(lmax), int(channels), F32, _ptr(x), _ptr(D),
                                           _ptr(weights), _ptr(grad_out), _ptr(grad_D), _ptr(workspace),
                                           workspace.numel() * workspace.element_size(), _stream_handle(stream)))
    return grad_D


@_on_launch_stream
def tpconv_so2_rotations_backward(lmax: int, vec, grad_D, grad_vec=None, stream=None) -> torch.Tensor:
    """grad_vec [E, 3] from grad_D [E, sum (2l+1)^2] (dtype of vec)."""
    E = vec.shape[0] if vec.dim() == 2 else -1
    dt = vec.dtype
    _need(vec, (E, 3), dt, "vec")
    nd = (lmax + 1) * (2 * lmax + 1) * (2 * lmax + 3) // 3
    _need(grad_D, (E, nd), dt, "grad_D")
    if grad_vec is None:
        grad_vec = torch.empty((E, 3), dtype=dt, device=vec.device)
    _need(grad_vec, (E, 3), dt, "grad_vec")
    _check(_lib.tpconv_so2_rotations_backward(int(lmax), F64 if dt == torch.float64 else F32, E, _ptr(vec),
                                              _ptr(grad_D), _ptr(grad_vec), _stream_handle(stream)))
    return grad_vec



@_on_launch_stream
def tpconv_so2_rotations_jvp(lmax: int, vec, dvec, dD=None, stream=None) -> torch.Tensor:
    """dD [E, sum (2l+1)^2]: the frames' derivative along dvec [E, 3] (dtype of vec)."""
    E = vec.shape[0] if vec.dim() == 2 else -1
    dt = vec.dtype
    _need(vec, (E, 3), dt, "vec")
    _need(dvec, (E, 3), dt, "dvec")
    nd = (lmax + 1) * (2 * lmax + 1) * (2 * lmax + 3) // 3
    if dD is None:
        dD = torch.empty((E, nd), dtype=dt, device=vec.device)
    _need(dD, (E, nd), dt, "dD")
    _check(_lib.tpconv_so2_rotations_jvp(int(lmax), F64 if dt == torch.float64 else F32, E, _ptr(vec), _ptr(dvec),
                                         _ptr(dD), _stream_handle(stream)))
    return dD


def tpconv_so2_frames_double_backward_workspace_bytes(lmax: int, channels: int, n_nodes: int, n_edges: int) -> int:
    return int(_lib.tpconv_so2_frames_double_backward_workspace_bytes(int(lmax), int(channels), int(n_nodes),
                                                                       int(n_edges)))


@_on_launch_stream
def tpconv_so2_frames_double_backward(graph: Graph, lmax: int, channels: int, x, D, weights, grad_out, dD,
                                      grad_x=None, grad_weights=None, grad_G=None, need=(True, True, True),
                                      workspace=None, stream=None):
    """(grad_x, grad_weights, grad_G) of <dD, tpconv_so2_frames_backward(...)>; None where `need` is off."""
    N, E = graph.n_nodes, graph.n_edges
    dn, nd, nw = _so2_sizes(lmax, channels)
    f = torch.float32
    _need(x, (N, dn), f, "x")
    _need(D, (E, nd), f, "D")
    _need(weights, (nw,), f, "weights")
    _need(grad_out, (N, dn), f, "grad_out")
    _need(dD, (E, nd), f, "dD")
    dev = x.device
    if need[0] and grad_x is None:
        grad_x = torch.empty((N, dn), dtype=f, device=dev)
    if need[1] and grad_weights is None:
        grad_weights = torch.empty((nw,), dtype=f, device=dev)
    if need[2] and grad_G is None:
        grad_G = torch.empty((N, dn), dtype=f, device=dev)
    for t, shape, name in ((grad_x, (N, dn), "grad_x"), (grad_weights, (nw,), "grad_weights"),
                           (grad_G, (N, dn), "grad_G")):
        if t is not None:
            _need(t, shape, f, name)
    if workspace is None:
        workspace = torch.empty(max(tpconv_so2_frames_double_backward_workspace_bytes(lmax, channels, N, E), 256),
                                dtype=torch.uint8, device=dev)
    _check(_lib.tpconv_so2_frames_double_backward(graph.handle, int(lmax), int(channels), F32, _ptr(x), _ptr(D),
                                                  _ptr(weights), _ptr(grad_out), _ptr(dD), _ptr(grad_x),
                                                  _ptr(grad_weights), _ptr(grad_G), _ptr(workspace),
                                                  workspace.numel() * workspace.element_size(),
                                                  _stream_handle(stream)))
    return grad_x, grad_weights, grad_G
