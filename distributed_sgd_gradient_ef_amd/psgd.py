"""Thin ctypes binding of libpsgd (C ABI declared in include/psgd.h,
include/psgd_rtopk.h and include/psgd_atomo.h).

Functions carry the C names.  The step functions take torch tensors on a ROCm device
and pass their device pointers and the current HIP stream; every step of the
computation runs in the library's HIP kernels.  Nothing here computes: if the library
is missing the import of a step function fails loudly.

Besides the C calls there are two layout helpers, ``pack`` and ``unpack``, which move
per-tensor arrays into and out of the plan's packed [workers][worker_stride] layout.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpsgd.so")

PSGD_OK = 0
PSGD_ERR_INVALID_ARG = 1
PSGD_ERR_UNSUPPORTED = 2
PSGD_ERR_NO_MEMORY = 3
PSGD_ERR_HIP = 4
PSGD_F32 = 0
PSGD_BF16 = 1
PSGD_FLAG_NESTEROV = 0x1
PSGD_FLAG_CARRY_ERROR_MEAN = 0x2
PSGD_FLAG_DEFERRED_ERROR = 0x4
PSGD_FLAG_LOCAL_Q_ERROR = 0x8
PSGD_RTOPK_FLAG_DEFERRED_ZERO = 0x1

EXPORTED = [
    "psgd_plan_create", "psgd_plan_sizes", "psgd_plan_layer_info", "psgd_plan_destroy",
    "psgd_compress_step", "psgd_compress_step_noalloc", "psgd_ef_momentum_apply", "psgd_plan_set_timing",
    "psgd_plan_kernel_stats", "psgd_plan_reset_carry", "psgd_plan_reset_carry_stream", "psgd_errors_materialize",
    "psgd_stream_copy",
    "psgd_plan_set_power_iterations", "psgd_status_string", "psgd_last_error",
    "psgd_rtopk_plan_create", "psgd_rtopk_plan_sizes", "psgd_rtopk_plan_layer_info", "psgd_rtopk_plan_destroy",
    "psgd_rtopk_step", "psgd_rtopk_plan_set_timing", "psgd_rtopk_plan_kernel_stats",
    "psgd_rtopk_errors_materialize", "psgd_rtopk_plan_reset_state",
    "psgd_atomo_plan_create", "psgd_atomo_plan_sizes", "psgd_atomo_plan_layer_info", "psgd_atomo_plan_destroy",
    "psgd_atomo_step", "psgd_atomo_plan_set_timing", "psgd_atomo_plan_kernel_stats",
]
PSGD_ATOMO_MAX_K = 1024
_STRING_FUNCS = ("psgd_status_string", "psgd_last_error")


class PsgdError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class _Layer(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


class _LayerInfo(ctypes.Structure):
    _fields_ = [("compressed", ctypes.c_int32), ("matrix_index", ctypes.c_int32),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("offset", ctypes.c_int64),
                ("p_offset", ctypes.c_int64), ("q_offset", ctypes.c_int64)]


class _KernelStat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double)]


class _Sizes(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("n_matrices", ctypes.c_int32),
                ("n_vectors", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("n_workers", ctypes.c_int32), ("grad_dtype", ctypes.c_int32),
                ("worker_stride", ctypes.c_int64), ("numel", ctypes.c_int64),
                ("matrix_numel", ctypes.c_int64), ("vector_numel", ctypes.c_int64),
                ("p_elems", ctypes.c_int64), ("q_elems", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_uint64), ("message_bytes", ctypes.c_uint64),
                ("model_bytes", ctypes.c_uint64), ("model_bytes_momentum", ctypes.c_uint64)]


class _RtopkLayerInfo(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("numel", ctypes.c_int64),
                ("offset", ctypes.c_int64), ("top", ctypes.c_int64), ("keep", ctypes.c_int64),
                ("top_offset", ctypes.c_int64), ("keep_offset", ctypes.c_int64)]


class _RtopkSizes(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("n_workers", ctypes.c_int32),
                ("grad_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("worker_stride", ctypes.c_int64), ("numel", ctypes.c_int64),
                ("top_total", ctypes.c_int64), ("keep_total", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_uint64), ("message_bytes", ctypes.c_uint64),
                ("model_bytes", ctypes.c_uint64)]


class _AtomoLayerInfo(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("numel", ctypes.c_int64),
                ("offset", ctypes.c_int64), ("compressed", ctypes.c_int32), ("matrix_index", ctypes.c_int32),
                ("k", ctypes.c_int64), ("sv_offset", ctypes.c_int64), ("atom_offset", ctypes.c_int64)]


class _AtomoSizes(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("n_workers", ctypes.c_int32),
                ("n_matrices", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("worker_stride", ctypes.c_int64), ("numel", ctypes.c_int64),
                ("sv_total", ctypes.c_int64), ("atom_total", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_uint64), ("model_bytes", ctypes.c_uint64),
                ("budget", ctypes.c_double)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpsgd.so (once).  Import torch first so the HIP runtime it carries is the
    one the library binds to (both use the soname libamdhip64.so.7)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m distributed_sgd_gradient_ef_amd.build`")
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    lib.psgd_plan_create.argtypes = [ctypes.POINTER(_Layer), i32, i32, i32, i32, ctypes.c_uint32,
                                     ctypes.POINTER(vp)]
    lib.psgd_plan_sizes.argtypes = [vp, ctypes.POINTER(_Sizes)]
    lib.psgd_plan_layer_info.argtypes = [vp, i32, ctypes.POINTER(_LayerInfo)]
    lib.psgd_plan_destroy.argtypes = [vp]
    lib.psgd_compress_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp]
    lib.psgd_compress_step_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    lib.psgd_ef_momentum_apply.argtypes = [vp, vp, vp, vp, vp, vp, vp, f32, f32, vp, vp, vp]
    lib.psgd_plan_set_timing.argtypes = [vp, i32]
    lib.psgd_plan_kernel_stats.argtypes = [vp, ctypes.POINTER(_KernelStat), i32, ctypes.POINTER(i32), i32]
    lib.psgd_plan_reset_carry.argtypes = [vp]
    lib.psgd_plan_reset_carry_stream.argtypes = [vp, vp, vp]
    lib.psgd_stream_copy.argtypes = [vp, vp, ctypes.c_uint64, vp]
    lib.psgd_errors_materialize.argtypes = [vp, vp, vp, vp, vp]
    lib.psgd_plan_set_power_iterations.argtypes = [vp, i32]
    i64p = ctypes.POINTER(i64)
    lib.psgd_rtopk_plan_create.argtypes = [ctypes.POINTER(_Layer), i32, i64p, i64p, i32, i32, ctypes.c_uint32,
                                           ctypes.POINTER(vp)]
    lib.psgd_rtopk_plan_sizes.argtypes = [vp, ctypes.POINTER(_RtopkSizes)]
    lib.psgd_rtopk_plan_layer_info.argtypes = [vp, i32, ctypes.POINTER(_RtopkLayerInfo)]
    lib.psgd_rtopk_plan_destroy.argtypes = [vp]
    lib.psgd_rtopk_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.psgd_rtopk_plan_set_timing.argtypes = [vp, i32]
    lib.psgd_rtopk_plan_kernel_stats.argtypes = [vp, ctypes.POINTER(_KernelStat), i32, ctypes.POINTER(i32), i32]
    lib.psgd_rtopk_errors_materialize.argtypes = [vp, vp, vp, vp, vp]
    lib.psgd_rtopk_plan_reset_state.argtypes = [vp, vp, vp]
    lib.psgd_atomo_plan_create.argtypes = [ctypes.POINTER(_Layer), i32, ctypes.c_double, i32, ctypes.c_uint32,
                                           ctypes.POINTER(vp)]
    lib.psgd_atomo_plan_sizes.argtypes = [vp, ctypes.POINTER(_AtomoSizes)]
    lib.psgd_atomo_plan_layer_info.argtypes = [vp, i32, ctypes.POINTER(_AtomoLayerInfo)]
    lib.psgd_atomo_plan_destroy.argtypes = [vp]
    lib.psgd_atomo_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.psgd_atomo_plan_set_timing.argtypes = [vp, i32]
    lib.psgd_atomo_plan_kernel_stats.argtypes = [vp, ctypes.POINTER(_KernelStat), i32, ctypes.POINTER(i32), i32]
    for name in EXPORTED:
        if name not in _STRING_FUNCS:
            getattr(lib, name).restype = ctypes.c_int
    lib.psgd_status_string.argtypes = [ctypes.c_int]
    lib.psgd_status_string.restype = ctypes.c_char_p
    lib.psgd_last_error.argtypes = []
    lib.psgd_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != PSGD_OK:
        lib = load_library()
        raise PsgdError(status, lib.psgd_last_error().decode() or lib.psgd_status_string(status).decode())


@dataclass
class LayerInfo:
    compressed: bool
    matrix_index: int
    rows: int
    cols: int
    offset: int
    p_offset: int
    q_offset: int


class Plan:
    """Owns a psgd_plan*; freed by psgd_plan_destroy (or when garbage collected)."""

    def __init__(self, handle: int, shapes: Sequence[Tuple[int, int]]):
        self.handle = handle
        self.shapes = [tuple(int(v) for v in s) for s in shapes]
        self.sizes = psgd_plan_sizes(self)
        self.layers: List[LayerInfo] = [psgd_plan_layer_info(self, i) for i in range(len(shapes))]

    def __del__(self):
        if getattr(self, "handle", None):
            try:
                psgd_plan_destroy(self)
            except Exception:
                pass


# ------------------------------------------------------------------------ C calls
def psgd_plan_create(shapes: Sequence[Tuple[int, int]], rank: int, n_workers: int,
                     grad_dtype: int = PSGD_F32, flags: int = 0) -> Plan:
    lib = load_library()
    arr = (_Layer * max(1, len(shapes)))(*[_Layer(int(r), int(c)) for r, c in shapes])
    h = ctypes.c_void_p()
    _check(lib.psgd_plan_create(arr, len(shapes), int(rank), int(n_workers), int(grad_dtype),
                                int(flags), ctypes.byref(h)))
    return Plan(h.value, shapes)


def psgd_plan_sizes(plan: Plan) -> dict:
    s = _Sizes()
    _check(load_library().psgd_plan_sizes(plan.handle, ctypes.byref(s)))
    return {name: getattr(s, name) for name, _ in _Sizes._fields_}


def psgd_plan_layer_info(plan: Plan, layer: int) -> LayerInfo:
    li = _LayerInfo()
    _check(load_library().psgd_plan_layer_info(plan.handle, int(layer), ctypes.byref(li)))
    return LayerInfo(bool(li.compressed), li.matrix_index, li.rows, li.cols, li.offset, li.p_offset,
                     li.q_offset)


def psgd_plan_destroy(plan: Plan) -> None:
    h, plan.handle = plan.handle, None
    if h:
        _check(load_library().psgd_plan_destroy(h))


def psgd_plan_set_timing(plan: Plan, enable: bool) -> None:
    _check(load_library().psgd_plan_set_timing(plan.handle, 1 if enable else 0))


def psgd_plan_kernel_stats(plan: Plan, reset: bool = False) -> dict:
    """{kernel name: (launches, total_ms)}; waits for every timed launch so far."""
    arr = (_KernelStat * 16)()
    n = ctypes.c_int32()
    _check(load_library().psgd_plan_kernel_stats(plan.handle, arr, 16, ctypes.byref(n), 1 if reset else 0))
    return {arr[i].name.decode(): (arr[i].launches, arr[i].total_ms) for i in range(n.value)}


def psgd_plan_set_power_iterations(plan: Plan, iterations: int) -> None:
    _check(load_library().psgd_plan_set_power_iterations(plan.handle, int(iterations)))


def psgd_plan_reset_carry(plan: Plan) -> None:
    _check(load_library().psgd_plan_reset_carry(plan.handle))


def psgd_plan_reset_carry_stream(plan: Plan, workspace, stream=None) -> None:
    """Stream-ordered reset of the cross-step state held in `workspace`."""
    import torch

    with torch.cuda.device(workspace.device):
        _check(load_library().psgd_plan_reset_carry_stream(plan.handle, _ptr(workspace),
                                                           _stream(stream, workspace)))


def psgd_errors_materialize(plan: Plan, errors, out, workspace, stream=None) -> None:
    """Plain error memory of a deferred-mode error buffer into `out` (may be `errors`)."""
    import torch

    with torch.cuda.device(errors.device):
        _check(load_library().psgd_errors_materialize(plan.handle, _ptr(errors), _ptr(out), _ptr(workspace),
                                                      _stream(stream, errors)))


def psgd_stream_copy(src, dst, nbytes: int, stream=None) -> None:
    """Calibration copy of `nbytes` from tensor `src` to tensor `dst` (same device)."""
    import torch

    with torch.cuda.device(src.device):
        _check(load_library().psgd_stream_copy(_ptr(src), _ptr(dst), int(nbytes), _stream(stream, src)))


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _stream(stream, ref):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(ref.device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream or 0)


def psgd_compress_step(plan: Plan, grads, errors, q, p, update, workspace, stream=None) -> None:
    """Enqueue one compression step (tensors on a ROCm device; see include/psgd.h)."""
    import torch

    with torch.cuda.device(grads.device):
        _check(load_library().psgd_compress_step(
            plan.handle, _ptr(grads), _ptr(errors), _ptr(q), _ptr(p), _ptr(update), _ptr(workspace),
            _stream(stream, grads)))


def psgd_compress_step_noalloc(plan: Plan, grads, errors, q, p, update, stream=None) -> None:
    """The same step with the workspace in the library's static device array (no
    device allocation; see include/psgd.h)."""
    import torch

    with torch.cuda.device(grads.device):
        _check(load_library().psgd_compress_step_noalloc(
            plan.handle, _ptr(grads), _ptr(errors), _ptr(q), _ptr(p), _ptr(update), _stream(stream, grads)))


def psgd_ef_momentum_apply(plan: Plan, grads, errors, q, p, momentum, params, lr: float, mu: float,
                           update, workspace, stream=None) -> None:
    """Enqueue one compression step fused with the momentum-SGD update."""
    import torch

    with torch.cuda.device(grads.device):
        _check(load_library().psgd_ef_momentum_apply(
            plan.handle, _ptr(grads), _ptr(errors), _ptr(q), _ptr(p), _ptr(momentum), _ptr(params),
            float(lr), float(mu), _ptr(update), _ptr(workspace), _stream(stream, grads)))


# ------------------------------------------------------------------------ rTop-k
@dataclass
class RtopkLayerInfo:
    rows: int
    cols: int
    numel: int
    offset: int
    top: int
    keep: int
    top_offset: int
    keep_offset: int


class RtopkPlan:
    """Owns a psgd_rtopk_plan*; freed by psgd_rtopk_plan_destroy (or when collected)."""

    def __init__(self, handle: int, shapes: Sequence[Tuple[int, int]]):
        self.handle = handle
        self.shapes = [tuple(int(v) for v in s) for s in shapes]
        self.sizes = psgd_rtopk_plan_sizes(self)
        self.layers: List[RtopkLayerInfo] = [psgd_rtopk_plan_layer_info(self, i) for i in range(len(shapes))]

    def __del__(self):
        if getattr(self, "handle", None):
            try:
                psgd_rtopk_plan_destroy(self)
            except Exception:
                pass


def psgd_rtopk_plan_create(shapes: Sequence[Tuple[int, int]], top: Sequence[int], keep: Sequence[int],
                           n_workers: int, grad_dtype: int = PSGD_F32, flags: int = 0) -> RtopkPlan:
    lib = load_library()
    n = len(shapes)
    arr = (_Layer * max(1, n))(*[_Layer(int(r), int(c)) for r, c in shapes])
    tops = (ctypes.c_int64 * max(1, n))(*[int(v) for v in top])
    keeps = (ctypes.c_int64 * max(1, n))(*[int(v) for v in keep])
    h = ctypes.c_void_p()
    _check(lib.psgd_rtopk_plan_create(arr, n, tops, keeps, int(n_workers), int(grad_dtype), int(flags),
                                      ctypes.byref(h)))
    return RtopkPlan(h.value, shapes)


def psgd_rtopk_plan_sizes(plan: RtopkPlan) -> dict:
    s = _RtopkSizes()
    _check(load_library().psgd_rtopk_plan_sizes(plan.handle, ctypes.byref(s)))
    return {name: getattr(s, name) for name, _ in _RtopkSizes._fields_}


def psgd_rtopk_plan_layer_info(plan: RtopkPlan, layer: int) -> RtopkLayerInfo:
    li = _RtopkLayerInfo()
    _check(load_library().psgd_rtopk_plan_layer_info(plan.handle, int(layer), ctypes.byref(li)))
    return RtopkLayerInfo(*(getattr(li, name) for name, _ in _RtopkLayerInfo._fields_))


def psgd_rtopk_plan_destroy(plan: RtopkPlan) -> None:
    h, plan.handle = plan.handle, None
    if h:
        _check(load_library().psgd_rtopk_plan_destroy(h))


def psgd_rtopk_plan_set_timing(plan: RtopkPlan, enable: bool) -> None:
    _check(load_library().psgd_rtopk_plan_set_timing(plan.handle, 1 if enable else 0))


def psgd_rtopk_plan_kernel_stats(plan: RtopkPlan, reset: bool = False) -> dict:
    """{kernel name: (launches, total_ms)}; waits for every timed launch so far."""
    arr = (_KernelStat * 16)()
    n = ctypes.c_int32()
    _check(load_library().psgd_rtopk_plan_kernel_stats(plan.handle, arr, 16, ctypes.byref(n), 1 if reset else 0))
    return {arr[i].name.decode(): (arr[i].launches, arr[i].total_ms) for i in range(n.value)}


def psgd_rtopk_step(plan: RtopkPlan, grads, errors, ranks, index, value, update, workspace, stream=None) -> None:
    """Enqueue one rTop-k step (tensors on a ROCm device; see include/psgd_rtopk.h)."""
    import torch

    with torch.cuda.device(grads.device):
        _check(load_library().psgd_rtopk_step(
            plan.handle, _ptr(grads), _ptr(errors), _ptr(ranks), _ptr(index), _ptr(value), _ptr(update),
            _ptr(workspace), _stream(stream, grads)))

def psgd_rtopk_errors_materialize(plan: RtopkPlan, errors, out, workspace, stream=None) -> None:
    """Plain error memory of a deferred-zero plan's error buffer into `out` (may be `errors`)."""
    import torch

    with torch.cuda.device(errors.device):
        _check(load_library().psgd_rtopk_errors_materialize(plan.handle, _ptr(errors), _ptr(out), _ptr(workspace),
                                                            _stream(stream, errors)))


def psgd_rtopk_plan_reset_state(plan: RtopkPlan, workspace, stream=None) -> None:
    """Forget the pending zeros of a deferred-zero plan (host view and, on the stream, the
    workspace's state word)."""
    import torch

    with torch.cuda.device(workspace.device):
        _check(load_library().psgd_rtopk_plan_reset_state(plan.handle, _ptr(workspace), _stream(stream, workspace)))


# ------------------------------------------------------------------------ Spectral-ATOMO
@dataclass
class AtomoLayerInfo:
    rows: int
    cols: int
    numel: int
    offset: int
    compressed: int
    matrix_index: int
    k: int
    sv_offset: int
    atom_offset: int


class AtomoPlan:
    """Owns a psgd_atomo_plan*; freed by psgd_atomo_plan_destroy (or when collected)."""

    def __init__(self, handle: int, shapes: Sequence[Tuple[int, int]]):
        self.handle = handle
        self.shapes = [tuple(int(v) for v in s) for s in shapes]
        self.sizes = psgd_atomo_plan_sizes(self)
        self.layers: List[AtomoLayerInfo] = [psgd_atomo_plan_layer_info(self, i) for i in range(len(shapes))]

    def __del__(self):
        if getattr(self, "handle", None):
            try:
                psgd_atomo_plan_destroy(self)
            except Exception:
                pass



def psgd_atomo_plan_create(shapes: Sequence[Tuple[int, int]], budget: float, n_workers: int,
                           flags: int = 0) -> AtomoPlan:
    lib = load_library()
    n = len(shapes)
    arr = (_Layer * max(1, n))(*[_Layer(int(r), int(c)) for r, c in shapes])
    h = ctypes.c_void_p()
    _check(lib.psgd_atomo_plan_create(arr, n, float(budget), int(n_workers), int(flags), ctypes.byref(h)))
    return AtomoPlan(h.value, shapes)


def psgd_atomo_plan_sizes(plan: AtomoPlan) -> dict:
    s = _AtomoSizes()
    _check(load_library().psgd_atomo_plan_sizes(plan.handle, ctypes.byref(s)))
    return {name: getattr(s, name) for name, _ in _AtomoSizes._fields_}


def psgd_atomo_plan_layer_info(plan: AtomoPlan, layer: int) -> AtomoLayerInfo:
    li = _AtomoLayerInfo()
    _check(load_library().psgd_atomo_plan_layer_info(plan.handle, int(layer), ctypes.byref(li)))
    return AtomoLayerInfo(*(getattr(li, name) for name, _ in _AtomoLayerInfo._fields_))


def psgd_atomo_plan_destroy(plan: AtomoPlan) -> None:
    h, plan.handle = plan.handle, None
    if h:
        _check(load_library().psgd_atomo_plan_destroy(h))


def psgd_atomo_plan_set_timing(plan: AtomoPlan, enable: bool) -> None:
    _check(load_library().psgd_atomo_plan_set_timing(plan.handle, 1 if enable else 0))


def psgd_atomo_plan_kernel_stats(plan: AtomoPlan, reset: bool = False) -> dict:
    """{kernel name: (launches, total_ms)}; waits for every timed launch so far."""
    arr = (_KernelStat * 16)()
    n = ctypes.c_int32()
    _check(load_library().psgd_atomo_plan_kernel_stats(plan.handle, arr, 16, ctypes.byref(n), 1 if reset else 0))
    return {arr[i].name.decode(): (arr[i].launches, arr[i].total_ms) for i in range(n.value)}


def psgd_atomo_step(plan: AtomoPlan, grads, uniforms, sigma, prob, index, count, atoms, update, workspace,
                    stream=None) -> None:
    """Enqueue one Spectral-ATOMO step (tensors on a ROCm device; see include/psgd_atomo.h)."""
    import torch

    with torch.cuda.device(grads.device):
        _check(load_library().psgd_atomo_step(
            plan.handle, _ptr(grads), _ptr(uniforms), _ptr(sigma), _ptr(prob), _ptr(index), _ptr(count),
            _ptr(atoms), _ptr(update), _ptr(workspace), _stream(stream, grads)))


def pack_sv(plan: AtomoPlan, per_layer: dict, dtype=np.float32) -> np.ndarray:
    """Place per-matrix (W, k) arrays ({layer: array}) into the [W][sv_total] rows of an
    ATOMO plan (zeros elsewhere)."""
    W = plan.sizes["n_workers"]
    out = np.zeros((W, plan.sizes["sv_total"]), dtype=dtype)
    for li, a in per_layer.items():
        L = plan.layers[li]
        out[:, L.sv_offset:L.sv_offset + L.k] = np.asarray(a).reshape(W, L.k)
    return out


def sv_slice(plan: AtomoPlan, rows: np.ndarray, layer: int) -> np.ndarray:
    """One matrix's (W, k) block of a [W][sv_total] array."""
    L = plan.layers[layer]
    return rows[:, L.sv_offset:L.sv_offset + L.k]


def atom_factors(plan: AtomoPlan, atoms: np.ndarray, count: np.ndarray, layer: int, worker: int):
    """The sent factors of one worker's matrix: (a [count, rows], b [count, cols])."""
    L = plan.layers[layer]
    cnt = int(count[worker, L.matrix_index])
    blk = atoms[worker, L.atom_offset:L.atom_offset + cnt * (L.rows + L.cols)].reshape(cnt, L.rows + L.cols)
    return blk[:, :L.rows], blk[:, L.rows:]


# ------------------------------------------------------------------------ layout helpers
def pack(plan, per_layer: Sequence[np.ndarray], dtype=np.float32, workers: Optional[int] = None,
         layers: Optional[Sequence[int]] = None) -> np.ndarray:
    """Place per-tensor arrays into the packed layout.

    per_layer[i] has shape (W, rows, cols) (or (rows, cols) when ``workers`` is 0, for
    update/momentum/params).  Returns (W, worker_stride) or (worker_stride,); padding is 0.
    """
    ld = plan.sizes["worker_stride"]
    W = plan.sizes["n_workers"] if workers is None else workers
    out = np.zeros((W, ld) if W else (ld,), dtype=dtype)
    idx = range(len(plan.layers)) if layers is None else layers
    for a, li in zip(per_layer, idx):
        L = plan.layers[li]
        n = L.rows * L.cols
        if W:
            out[:, L.offset:L.offset + n] = np.asarray(a).reshape(W, n)
        else:
            out[L.offset:L.offset + n] = np.asarray(a).reshape(n)
    return out


def unpack(plan, flat: np.ndarray, layer: int) -> np.ndarray:
    """Inverse of ``pack`` for one tensor: (W, rows, cols) or (rows, cols)."""
    L = plan.layers[layer]
    n = L.rows * L.cols
    if flat.ndim == 2:
        return flat[:, L.offset:L.offset + n].reshape(flat.shape[0], L.rows, L.cols)
    return flat[L.offset:L.offset + n].reshape(L.rows, L.cols)


def factor_slice(plan: Plan, flat: np.ndarray, layer: int, which: str) -> np.ndarray:
    """P (rows x rank) or Q (cols x rank) of one compressed matrix from the flat p or q."""
    L = plan.layers[layer]
    r = plan.sizes["rank"]
    if which == "p":
        return flat[L.p_offset:L.p_offset + L.rows * r].reshape(L.rows, r)
    return flat[L.q_offset:L.q_offset + L.cols * r].reshape(L.cols, r)


def pack_factors(plan: Plan, per_matrix: dict, which: str) -> np.ndarray:
    """Concatenate per-layer P or Q arrays ({layer: array}) into the flat p or q buffer."""
    r = plan.sizes["rank"]
    n = plan.sizes["p_elems" if which == "p" else "q_elems"]
    out = np.zeros(n, dtype=np.float32)
    for li, a in per_matrix.items():
        L = plan.layers[li]
        off = L.p_offset if which == "p" else L.q_offset
        k = (L.rows if which == "p" else L.cols) * r
        out[off:off + k] = np.asarray(a, dtype=np.float32).reshape(k)
    return out


def pack_rows(plan: RtopkPlan, per_layer: Sequence[np.ndarray], which: str, dtype) -> np.ndarray:
    """Concatenate per-tensor (W, top) or (W, keep) arrays into the [W][top_total] or
    [W][keep_total] rows of an rTop-k plan."""
    W = plan.sizes["n_workers"]
    total = plan.sizes["top_total" if which == "top" else "keep_total"]
    out = np.zeros((W, total), dtype=dtype)
    for a, L in zip(per_layer, plan.layers):
        off, n = (L.top_offset, L.top) if which == "top" else (L.keep_offset, L.keep)
        out[:, off:off + n] = np.asarray(a).reshape(W, n)
    return out


def row_slice(plan: RtopkPlan, rows: np.ndarray, layer: int, which: str) -> np.ndarray:
    """One tensor's (W, top) or (W, keep) block of a [W][total] row array."""
    L = plan.layers[layer]
    off, n = (L.top_offset, L.top) if which == "top" else (L.keep_offset, L.keep)
    return rows[:, off:off + n]
