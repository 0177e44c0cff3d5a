"""Python binding of libqgemv (include/qgemv.h): argument marshalling only.

Every function has the name and the meaning of the C entry point it calls; all work runs in
the library's HIP kernels on the GPU. torch supplies device memory (tensors) and streams; the
library is loaded after torch so that both share torch's HIP runtime. There is no fallback:
if the library is not built, importing a function raises.

Tensors must be CUDA (HIP) tensors, contiguous, with the dtypes the C ABI names; they are
passed as raw device pointers. `stream=None` means torch's current stream on the tensor's
device.
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "QGEMV_Q4K", "QGEMV_Q6K", "QgemvError", "library_path", "qgemv_version",
    "qgemv_status_string", "qgemv_weight_bytes", "qgemv_quantize_act",
    "qgemv_workspace_bytes", "qgemv_q4k", "qgemv_q6k", "qgemv_batch", "qgemv_batch_scratch", "qgemv_debug_partials",
    "qgemv_quantize_weights", "qgemv_plan_for", "qgemv_plan_workspace_bytes", "qgemv_batch_plan",
    "qgemv_read_probe", "qgemv_fused", "qgemv_fused_plan", "qgemv_quantize_weights_rows", "qgemv_fused_launches",
    "qgemv_multi", "qgemv_multi_fused", "qgemv_multi_geometry", "QGEMV_Q4_0", "QGEMV_Q8_0",
    "Graph", "qgemv_graph_begin", "qgemv_graph_end", "qgemv_graph_launch", "qgemv_graph_nodes",
    "qgemv_graph_destroy", "qgemv_graph_classify", "qgemv_i8mc_workspace_bytes", "qgemv_batch_i8mc",
    "qgemv_mc32_workspace_bytes", "qgemv_batch_mc32", "qgemv_debug_partials_mc32",
    "qgemv_mc32_tile",
    "qgemv_debug_partials_i8mc", "qgemv_fused_i8mc", "qgemv_route", "ROUTES",
]

QGEMV_Q4K = 1
QGEMV_Q6K = 2
QGEMV_Q4_0 = 3
QGEMV_Q8_0 = 4
WTYPES = {"q4k": QGEMV_Q4K, "q6k": QGEMV_Q6K, "q40": QGEMV_Q4_0, "q80": QGEMV_Q8_0}

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "_lib", "libqgemv.so")


class QgemvError(RuntimeError):
    def __init__(self, fn: str, status: int, lib):
        msg = lib.qgemv_status_string(status).decode()
        if status == 4:
            msg += ": " + lib.qgemv_last_error().decode()
        super().__init__("%s failed with status %d (%s)" % (fn, status, msg))
        self.status = status


class Plan(ctypes.Structure):
    _fields_ = [("lanes_per_row", ctypes.c_int32), ("chunks_per_lane", ctypes.c_int32),
                ("waves_per_block", ctypes.c_int32), ("blocks", ctypes.c_int32),
                ("splits", ctypes.c_int32)]

    def as_dict(self):
        return {name: int(getattr(self, name)) for name, _ in self._fields_}


class Matrix(ctypes.Structure):
    """One matrix of qgemv_multi / qgemv_multi_fused (the ABI's qgemv_matrix)."""
    _fields_ = [("wtype", ctypes.c_int32), ("reserved", ctypes.c_int32), ("rows", ctypes.c_int64),
                ("w", ctypes.c_void_p), ("y", ctypes.c_void_p)]


MAX_MATRICES = 8

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise RuntimeError("libqgemv.so is not built (%s); run __graft_entry__.build()" % library_path)
    lib = ctypes.CDLL(library_path)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    sigs = {
        "qgemv_version": (ctypes.c_int, []),
        "qgemv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "qgemv_last_error": (ctypes.c_char_p, []),
        "qgemv_weight_bytes": (sz, [ctypes.c_int, i64, i64]),
        "qgemv_quantize_act": (ctypes.c_int, [vp, vp, vp, i64, i32, vp]),
        "qgemv_workspace_bytes": (sz, [ctypes.c_int, i64, i64, i32]),
        "qgemv_q4k": (ctypes.c_int, [vp, vp, vp, vp, i64, i64, vp, sz, vp]),
        "qgemv_q6k": (ctypes.c_int, [vp, vp, vp, vp, i64, i64, vp, sz, vp]),
        "qgemv_batch": (ctypes.c_int, [ctypes.c_int, vp, vp, vp, vp, i64, i64, i32, vp, sz, vp]),
        "qgemv_batch_scratch": (ctypes.c_int, [ctypes.c_int, vp, vp, vp, vp, i64, i64, i32, vp]),
        "qgemv_debug_partials": (ctypes.c_int, [ctypes.c_int, vp, vp, vp, vp, vp, i64, i64, i32, vp,
                                                sz, vp]),
        "qgemv_quantize_weights": (ctypes.c_int, [ctypes.c_int, vp, vp, i64, i64, vp]),
        "qgemv_quantize_weights_rows": (ctypes.c_int, [ctypes.c_int, vp, vp, i64, i64, i64, i64, vp]),
        "qgemv_fused_launches": (ctypes.c_int, [ctypes.c_int, i64, i64, i32, ctypes.c_int]),
        "qgemv_multi": (ctypes.c_int, [ctypes.POINTER(Matrix), i32, vp, vp, i64, i32, vp]),
        "qgemv_multi_geometry": (ctypes.c_int, [i64, i32, ctypes.POINTER(ctypes.c_int32),
                                                ctypes.POINTER(ctypes.c_int32)]),
        "qgemv_multi_fused": (ctypes.c_int, [ctypes.POINTER(Matrix), i32, vp, vp, vp, i64, i32, vp]),
        "qgemv_plan_for": (ctypes.c_int, [ctypes.c_int, i64, i64, i32, ctypes.POINTER(Plan)]),
        "qgemv_plan_workspace_bytes": (sz, [ctypes.POINTER(Plan), i64, i64, i32]),
        "qgemv_batch_plan": (ctypes.c_int, [ctypes.c_int, vp, vp, vp, vp, i64, i64, i32,
                                            ctypes.POINTER(Plan), vp, sz, vp]),
        "qgemv_read_probe": (ctypes.c_int, [vp, sz, vp, i32, vp]),
        "qgemv_fused_plan": (ctypes.c_int, [ctypes.c_int, vp, vp, vp, vp, vp, i64, i64, i32,
                                            ctypes.POINTER(Plan), vp, sz, vp]),
        "qgemv_fused": (ctypes.c_int, [ctypes.c_int, vp, vp, vp, vp, vp, i64, i64, i32, vp, sz, vp]),
        "qgemv_graph_begin": (ctypes.c_int, [vp]),
        "qgemv_graph_end": (ctypes.c_int, [vp, ctypes.POINTER(vp)]),
        "qgemv_graph_launch": (ctypes.c_int, [vp, vp]),
        "qgemv_graph_nodes": (ctypes.c_int, [vp, ctypes.POINTER(i64), ctypes.POINTER(i64)]),
        "qgemv_graph_destroy": (ctypes.c_int, [vp]),
        "qgemv_graph_classify": (ctypes.c_int, [ctypes.POINTER(i32), i64, ctypes.POINTER(i64),
                                                ctypes.POINTER(i64)]),
        "qgemv_i8mc_workspace_bytes": (sz, [i64, i64, i32]),
        "qgemv_route": (ctypes.c_int, [ctypes.c_int, i64, i64, i32]),
        "qgemv_batch_i8mc": (ctypes.c_int, [vp, vp, vp, vp, i64, i64, i32, vp, sz, vp]),
        "qgemv_mc32_workspace_bytes": (sz, [i32, i64, i64, i32]),
        "qgemv_batch_mc32": (ctypes.c_int, [i32, vp, vp, vp, vp, i64, i64, i32, vp, sz, vp]),
        "qgemv_debug_partials_i8mc": (ctypes.c_int, [vp, vp, vp, vp, vp, i64, i64, i32, vp]),
        "qgemv_debug_partials_mc32": (ctypes.c_int, [i32, vp, vp, vp, vp, vp, i64, i64, i32, vp]),
        "qgemv_mc32_tile": (ctypes.c_int, [i32, i64, i64, i32]),
        "qgemv_fused_i8mc": (ctypes.c_int, [vp, vp, vp, vp, vp, i64, i64, i32, vp, sz, vp]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor or a device pointer" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor, got %s" % (name, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    return t.data_ptr()


def _stream(stream, *tensors):
    if stream is None:
        dev = next((t.device for t in tensors if isinstance(t, torch.Tensor)), None)
        return torch.cuda.current_stream(dev).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _nbytes(t):
    return t.numel() * t.element_size() if isinstance(t, torch.Tensor) else None


def _check(fn, status):
    if status != 0:
        raise QgemvError(fn, status, _load())


def _wtype(wtype):
    return WTYPES[wtype] if isinstance(wtype, str) else int(wtype)


def _ws(workspace):
    if workspace is None:
        return None, 0
    return _ptr(workspace, name="workspace"), _nbytes(workspace) or 0


# ------------------------------------------------------------------ info --
def qgemv_version() -> int:
    return _load().qgemv_version()


def qgemv_status_string(status: int) -> str:
    return _load().qgemv_status_string(status).decode()


def qgemv_weight_bytes(wtype, rows: int, cols: int) -> int:
    return _load().qgemv_weight_bytes(_wtype(wtype), rows, cols)


def qgemv_workspace_bytes(wtype, rows: int, cols: int, nvec: int = 1) -> int:
    return _load().qgemv_workspace_bytes(_wtype(wtype), rows, cols, nvec)


def qgemv_plan_for(wtype, rows: int, cols: int, nvec: int = 1) -> dict:
    plan = Plan()
    _check("qgemv_plan_for", _load().qgemv_plan_for(_wtype(wtype), rows, cols, nvec,
                                                   ctypes.byref(plan)))
    return plan.as_dict()


def qgemv_plan_workspace_bytes(plan: dict, rows: int, cols: int, nvec: int = 1) -> int:
    p = Plan(**{k: v for k, v in plan.items() if k in dict(Plan._fields_)})
    return _load().qgemv_plan_workspace_bytes(ctypes.byref(p), rows, cols, nvec)


# ------------------------------------------------------------- compute --
def qgemv_quantize_act(x, xq, xd, cols: int, nvec: int = 1, stream=None) -> None:
    """x float32 [nvec][cols] -> xq int8 [nvec][cols], xd float32 [nvec][cols/32]."""
    lib = _load()
    _check("qgemv_quantize_act", lib.qgemv_quantize_act(
        _ptr(x, torch.float32, "x"), _ptr(xq, torch.int8, "xq"), _ptr(xd, torch.float32, "xd"),
        cols, nvec, _stream(stream, x)))


def qgemv_q4k(w, xq, xd, y, rows: int, cols: int, workspace=None, stream=None) -> None:
    lib = _load()
    wsp, wsb = _ws(workspace)
    _check("qgemv_q4k", lib.qgemv_q4k(
        _ptr(w, name="w"), _ptr(xq, torch.int8, "xq"), _ptr(xd, torch.float32, "xd"),
        _ptr(y, torch.float32, "y"), rows, cols, wsp, wsb, _stream(stream, y)))


def qgemv_q6k(w, xq, xd, y, rows: int, cols: int, workspace=None, stream=None) -> None:
    lib = _load()
    wsp, wsb = _ws(workspace)
    _check("qgemv_q6k", lib.qgemv_q6k(
        _ptr(w, name="w"), _ptr(xq, torch.int8, "xq"), _ptr(xd, torch.float32, "xd"),
        _ptr(y, torch.float32, "y"), rows, cols, wsp, wsb, _stream(stream, y)))


def qgemv_batch(wtype, w, xq, xd, y, rows: int, cols: int, nvec: int, workspace=None,
                stream=None) -> None:
    lib = _load()
    wsp, wsb = _ws(workspace)
    _check("qgemv_batch", lib.qgemv_batch(
        _wtype(wtype), _ptr(w, name="w"), _ptr(xq, torch.int8, "xq"),
        _ptr(xd, torch.float32, "xd"), _ptr(y, torch.float32, "y"), rows, cols, nvec, wsp, wsb,
        _stream(stream, y)))


def qgemv_batch_scratch(wtype, w, xq, xd, y, rows: int, cols: int, nvec: int,
                        stream=None) -> None:
    """qgemv_batch with the library's static device scratch as its workspace (no workspace
    argument; nothing allocated)."""
    _check("qgemv_batch_scratch", _load().qgemv_batch_scratch(
        _wtype(wtype), _ptr(w, name="w"), _ptr(xq, torch.int8, "xq"),
        _ptr(xd, torch.float32, "xd"), _ptr(y, torch.float32, "y"), rows, cols, nvec,
        _stream(stream, y)))


SCRATCH_BYTES = 32 << 20       # the header's QGEMV_SCRATCH_BYTES


def qgemv_batch_plan(wtype, w, xq, xd, y, rows: int, cols: int, nvec: int, plan: dict,
                     workspace=None, stream=None) -> None:
    lib = _load()
    wsp, wsb = _ws(workspace)
    p = Plan(**{k: v for k, v in plan.items() if k in dict(Plan._fields_)})
    _check("qgemv_batch_plan", lib.qgemv_batch_plan(
        _wtype(wtype), _ptr(w, name="w"), _ptr(xq, torch.int8, "xq"),
        _ptr(xd, torch.float32, "xd"), _ptr(y, torch.float32, "y"), rows, cols, nvec,
        ctypes.byref(p), wsp, wsb, _stream(stream, y)))


def qgemv_fused(wtype, w, x, y, rows: int, cols: int, nvec: int, xq_out=None, xd_out=None,
                workspace=None, stream=None) -> None:
    """Quantize x (float32 [nvec][cols]) and compute y = W x in one launch; xq_out / xd_out
    optionally receive the codes and scales."""
    lib = _load()
    wsp, wsb = _ws(workspace)
    _check("qgemv_fused", lib.qgemv_fused(
        _wtype(wtype), _ptr(w, name="w"), _ptr(x, torch.float32, "x"),
        _ptr(xq_out, torch.int8, "xq_out"), _ptr(xd_out, torch.float32, "xd_out"),
        _ptr(y, torch.float32, "y"), rows, cols, nvec, wsp, wsb, _stream(stream, y)))


def qgemv_fused_plan(wtype, w, x, y, rows: int, cols: int, nvec: int, plan: dict, xq_out=None,
                     xd_out=None, workspace=None, stream=None) -> None:
    """qgemv_fused with an explicit plan: always the one-launch fused kernel (plus the
    ordered reduce when the plan splits the columns)."""
    lib = _load()
    wsp, wsb = _ws(workspace)
    p = Plan(**{k: v for k, v in plan.items() if k in dict(Plan._fields_)})
    _check("qgemv_fused_plan", lib.qgemv_fused_plan(
        _wtype(wtype), _ptr(w, name="w"), _ptr(x, torch.float32, "x"),
        _ptr(xq_out, torch.int8, "xq_out"), _ptr(xd_out, torch.float32, "xd_out"),
        _ptr(y, torch.float32, "y"), rows, cols, nvec, ctypes.byref(p), wsp, wsb,
        _stream(stream, y)))


def _matrices(mats):
    """[(wtype, w, rows, y), ...] -> a ctypes array of Matrix."""
    arr = (Matrix * max(1, len(mats)))()
    for i, (wtype, w, rows, y) in enumerate(mats):
        arr[i] = Matrix(_wtype(wtype), 0, rows, _ptr(w, name="w"), _ptr(y, torch.float32, "y"))
    return arr


def qgemv_multi_geometry(cols: int, nvec: int = 1) -> tuple:
    """(lanes_per_row, chunks_per_lane) of a multi-matrix launch for this row width."""
    t, nc = ctypes.c_int32(), ctypes.c_int32()
    _check("qgemv_multi_geometry", _load().qgemv_multi_geometry(cols, nvec, ctypes.byref(t),
                                                               ctypes.byref(nc)))
    return t.value, nc.value


def qgemv_multi(mats, xq, xd, cols: int, nvec: int = 1, stream=None) -> None:
    """y_m = W_m x for every (wtype, w, rows, y) in mats, one launch, from codes and scales."""
    lib = _load()
    _check("qgemv_multi", lib.qgemv_multi(
        _matrices(mats), len(mats), _ptr(xq, torch.int8, "xq"), _ptr(xd, torch.float32, "xd"),
        cols, nvec, _stream(stream, xq)))


def qgemv_multi_fused(mats, x, cols: int, nvec: int = 1, xq_out=None, xd_out=None,
                      stream=None) -> None:
    """The same from the float32 activation, quantized inside."""
    lib = _load()
    _check("qgemv_multi_fused", lib.qgemv_multi_fused(
        _matrices(mats), len(mats), _ptr(x, torch.float32, "x"),
        _ptr(xq_out, torch.int8, "xq_out"), _ptr(xd_out, torch.float32, "xd_out"), cols, nvec,
        _stream(stream, x)))


def qgemv_debug_partials(wtype, w, xq, xd, P, S, rows: int, cols: int, nvec: int = 1,
                         workspace=None, stream=None) -> None:
    lib = _load()
    wsp, wsb = _ws(workspace)
    _check("qgemv_debug_partials", lib.qgemv_debug_partials(
        _wtype(wtype), _ptr(w, name="w"), _ptr(xq, torch.int8, "xq"),
        _ptr(xd, torch.float32, "xd"), _ptr(P, torch.int32, "P"), _ptr(S, torch.int32, "S"),
        rows, cols, nvec, wsp, wsb, _stream(stream, P)))


ROUTES = {1: "vector", 2: "i8mc", 3: "mc", 4: "grouped", 5: "mc32"}


def qgemv_route(wtype, rows: int, cols: int, nvec: int = 1) -> str:
    """Which kernels qgemv_batch runs for this shape: "vector", "i8mc" (integer matrix cores),
    "mc" (float matrix cores, 17+ Q4_K vectors), "mc32" (integer matrix cores, 9+ Q8_0 / Q4_0 /
    Q6_K vectors) or "grouped" (vector kernels on groups of 8)."""
    lib = _load()
    r = int(lib.qgemv_route(_wtype(wtype), rows, cols, nvec))
    if r not in ROUTES:
        raise QgemvError("qgemv_route", 1, lib)
    return ROUTES[r]


def qgemv_i8mc_workspace_bytes(rows: int, cols: int, nvec: int) -> int:
    return int(_load().qgemv_i8mc_workspace_bytes(rows, cols, nvec))


def qgemv_batch_i8mc(w, xq, xd, y, rows: int, cols: int, nvec: int, workspace=None,
                     stream=None) -> None:
    """Q4_K y = W x for 1..8 vectors on the integer matrix cores, whatever the shape."""
    lib = _load()
    wsp, wsb = _ws(workspace)
    _check("qgemv_batch_i8mc", lib.qgemv_batch_i8mc(
        _ptr(w, name="w"), _ptr(xq, torch.int8, "xq"), _ptr(xd, torch.float32, "xd"),
        _ptr(y, torch.float32, "y"), rows, cols, nvec, wsp, wsb, _stream(stream, y)))


def qgemv_mc32_workspace_bytes(wtype, rows: int, cols: int, nvec: int) -> int:
    return int(_load().qgemv_mc32_workspace_bytes(_wtype(wtype), rows, cols, nvec))


def qgemv_batch_mc32(wtype, w, xq, xd, y, rows: int, cols: int, nvec: int, workspace=None,
                     stream=None) -> None:
    """Q8_0 / Q4_0 / Q6_K y = W x for 9..256 vectors (Q8_0 / Q4_0 also 1..8) on the integer
    matrix cores, whatever the shape."""
    lib = _load()
    wsp, wsb = _ws(workspace)
    _check("qgemv_batch_mc32", lib.qgemv_batch_mc32(
        _wtype(wtype), _ptr(w, name="w"), _ptr(xq, torch.int8, "xq"),
        _ptr(xd, torch.float32, "xd"), _ptr(y, torch.float32, "y"), rows, cols, nvec, wsp, wsb,
        _stream(stream, y)))


def qgemv_mc32_tile(wtype, rows: int, cols: int, nvec: int) -> int:
    """16 or 32: the kernel qgemv_batch_mc32 runs for the shape (0: not taken)."""
    return int(_load().qgemv_mc32_tile(_wtype(wtype), rows, cols, nvec))


def qgemv_debug_partials_mc32(wtype, w, xq, xd, P, S, rows: int, cols: int, nvec: int,
                              stream=None) -> None:
    lib = _load()
    _check("qgemv_debug_partials_mc32", lib.qgemv_debug_partials_mc32(
        _wtype(wtype), _ptr(w, name="w"), _ptr(xq, torch.int8, "xq"),
        _ptr(xd, torch.float32, "xd"), _ptr(P, torch.int32, "P"), _ptr(S, torch.int32, "S"),
        rows, cols, nvec, _stream(stream, P)))


def qgemv_debug_partials_i8mc(w, xq, xd, P, S, rows: int, cols: int, nvec: int,
                              stream=None) -> None:
    lib = _load()
    _check("qgemv_debug_partials_i8mc", lib.qgemv_debug_partials_i8mc(
        _ptr(w, name="w"), _ptr(xq, torch.int8, "xq"), _ptr(xd, torch.float32, "xd"),
        _ptr(P, torch.int32, "P"), _ptr(S, torch.int32, "S"), rows, cols, nvec,
        _stream(stream, P)))


def qgemv_fused_i8mc(w, x, y, rows: int, cols: int, nvec: int, xq_out=None, xd_out=None,
                     workspace=None, stream=None) -> None:
    lib = _load()
    wsp, wsb = _ws(workspace)
    _check("qgemv_fused_i8mc", lib.qgemv_fused_i8mc(
        _ptr(w, name="w"), _ptr(x, torch.float32, "x"), _ptr(xq_out, torch.int8, "xq_out"),
        _ptr(xd_out, torch.float32, "xd_out"), _ptr(y, torch.float32, "y"), rows, cols, nvec,
        wsp, wsb, _stream(stream, y)))


def qgemv_quantize_weights(wtype, w, out, rows: int, cols: int, stream=None) -> None:
    lib = _load()
    _check("qgemv_quantize_weights", lib.qgemv_quantize_weights(
        _wtype(wtype), _ptr(w, torch.float32, "w"), _ptr(out, name="out"), rows, cols,
        _stream(stream, out)))


def qgemv_fused_launches(wtype, rows: int, cols: int, nvec: int = 1,
                         with_outputs: bool = True) -> int:
    """1 or 2: the kernel launches qgemv_fused makes for this shape."""
    n = _load().qgemv_fused_launches(_wtype(wtype), rows, cols, nvec, int(bool(with_outputs)))
    if n == 0:
        raise ValueError("invalid weight type or shape")
    return n


def qgemv_quantize_weights_rows(wtype, w, out, rows: int, cols: int, row0: int, nrows: int,
                                stream=None) -> None:
    """Rows [row0, row0 + nrows) (w: float32 [nrows][cols]) into their places in the whole
    rows x cols tensor `out`."""
    lib = _load()
    _check("qgemv_quantize_weights_rows", lib.qgemv_quantize_weights_rows(
        _wtype(wtype), _ptr(w, torch.float32, "w"), _ptr(out, name="out"), rows, cols, row0,
        nrows, _stream(stream, out)))


def qgemv_read_probe(buf, sink, blocks: int = 2048, nbytes: int | None = None, stream=None) -> None:
    """Read `nbytes` (default: all) of `buf` once; a measurement of the read ceiling."""
    lib = _load()
    n = _nbytes(buf) if nbytes is None else nbytes
    _check("qgemv_read_probe", lib.qgemv_read_probe(_ptr(buf, name="buf"), n, _ptr(sink, name="sink"),
                                                    blocks, _stream(stream, buf)))


# ---------------------------------------------------------------- graphs --
class Graph:
    """A captured sequence of library calls (qgemv_graph_end); launch() replays it."""

    def __init__(self, handle: int):
        self._h = handle

    def launch(self, stream=None) -> None:
        if not self._h:
            raise ValueError("graph is closed")
        _check("qgemv_graph_launch", _load().qgemv_graph_launch(self._h, _stream(stream)))

    def nodes(self) -> tuple:
        """(kernel launches, other nodes) recorded in the graph."""
        k, o = ctypes.c_int64(), ctypes.c_int64()
        _check("qgemv_graph_nodes", _load().qgemv_graph_nodes(self._h, ctypes.byref(k),
                                                               ctypes.byref(o)))
        return k.value, o.value

    def close(self) -> None:
        """Free the graph; its last launch must have finished."""
        if self._h:
            _load().qgemv_graph_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def qgemv_graph_begin(stream=None) -> None:
    """Start recording this library's calls on `stream` (a created stream, default: the
    current one)."""
    _check("qgemv_graph_begin", _load().qgemv_graph_begin(_stream(stream)))


def qgemv_graph_end(stream=None) -> Graph:
    """Stop recording on `stream` and return the recorded calls as a Graph."""
    h = ctypes.c_void_p()
    _check("qgemv_graph_end", _load().qgemv_graph_end(_stream(stream), ctypes.byref(h)))
    return Graph(h.value)


def qgemv_graph_launch(graph: Graph, stream=None) -> None:
    graph.launch(stream)


def qgemv_graph_nodes(graph: Graph) -> tuple:
    return graph.nodes()


def qgemv_graph_destroy(graph: Graph) -> None:
    graph.close()


def qgemv_graph_classify(types) -> tuple:
    """(kernel nodes, other nodes) of a record with these HIP graph node types, as
    qgemv_graph_end counts them; QgemvError when one of them is a memset node. Host only."""
    arr = (ctypes.c_int32 * max(1, len(types)))(*[int(t) for t in types])
    k, o = ctypes.c_int64(), ctypes.c_int64()
    _check("qgemv_graph_classify",
           _load().qgemv_graph_classify(arr, len(types), ctypes.byref(k), ctypes.byref(o)))
    return int(k.value), int(o.value)
