"""ctypes binding of libtilepipe (the C ABI in include/tilepipe.h).

Argument marshalling only: every step of every operation runs in the HIP
kernels of ``libtilepipe.so``. torch provides device memory and the stream.
The library is loaded on first use; if it has not been built the call raises
(there is no CPU fallback).
"""
from __future__ import annotations

import ctypes
import enum
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libtilepipe.so")

_STATUS = ["TP_OK", "TP_ERR_INVALID_ARG", "TP_ERR_MISALIGNED", "TP_ERR_LDS_BUDGET",
           "TP_ERR_OVERLAP", "TP_ERR_UNSUPPORTED_DEVICE", "TP_ERR_HIP"]
OPS = {"scale2": 0, "horner32": 1, "copy": 2}


class Path(enum.IntEnum):
    X4 = 0
    SCALAR_LOAD = 1
    SCALAR_STORE = 2
    SCALAR = 3


class Schedule(enum.IntEnum):
    UNIFORM = 0
    ROLE_SPLIT = 1


class Align(enum.IntEnum):
    REALIGN = 0
    WORDS = 1


def _align(align) -> int:
    """tp_align value for the C ABI; out-of-range integers pass through so the
    library reports them."""
    if isinstance(align, str):
        try:
            return int(Align[align.upper()])
        except KeyError:
            raise ValueError(f"unknown align {align!r}; expected 'realign' or 'words'")
    return int(align)


def _schedule(schedule) -> int:
    """Schedule value for the C ABI; out-of-range integers pass through so the
    library reports them."""
    if isinstance(schedule, str):
        try:
            return int(Schedule[schedule.upper()])
        except KeyError:
            raise ValueError(f"unknown schedule {schedule!r}; expected 'uniform' or 'role_split'")
    return int(schedule)


class TilepipeError(RuntimeError):
    def __init__(self, status: int, where: str = "", hip_error: int = 0):
        self.status = status
        self.hip_error = hip_error
        name = _STATUS[status] if 0 <= status < len(_STATUS) else f"status {status}"
        msg = f"{where}: {name}" if where else name
        if hip_error:
            msg += f" (hipError_t {hip_error})"
        super().__init__(msg)


class _CPlan(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("stages", ctypes.c_int32),
                ("tile_units", ctypes.c_int32), ("threads", ctypes.c_int32),
                ("lane_chunks", ctypes.c_int32), ("tiles_per_block", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int32), ("wait_steady", ctypes.c_int32),
                ("num_tiles", ctypes.c_int64), ("grid", ctypes.c_int64),
                ("ring_bytes", ctypes.c_int32), ("resident_cap", ctypes.c_int32),
                ("schedule", ctypes.c_int32), ("chunk_bytes", ctypes.c_int32),
                ("align", ctypes.c_int32), ("head", ctypes.c_int32)]


@dataclass(frozen=True)
class Plan:
    path: Path
    stages: int
    tile_units: int
    threads: int
    lane_chunks: int
    tiles_per_block: int
    lds_bytes: int
    wait_steady: int
    num_tiles: int
    grid: int
    ring_bytes: int
    resident_cap: int
    schedule: "Schedule"
    chunk_bytes: int
    align: "Align"
    head: int


_lib = None


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is not built; run `python -m software_pipelining_amd.build` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    ip = ctypes.POINTER(ctypes.c_int)
    pp = ctypes.POINTER(_CPlan)
    sig = {
        "tp_status_string": ([i32], ctypes.c_char_p),
        "tp_last_hip_error": ([], i32),
        "tp_version": ([], i32),
        "tp_device_check": ([i32], i32),
        "tp_device_lds_budget": ([i32, ctypes.POINTER(ctypes.c_int64)], i32),
        "tp_row_shift": ([vp, vp, i64, vp, ip], i32),
        "tp_pipelined_map": ([vp, vp, i64, i32, i32, i32, i32, vp, ip], i32),
        "tp_pipelined_map_ex": ([vp, vp, i64, i32, i32, i32, i32, i32, i32, i32, vp, ip], i32),
        "tp_chunk_copy": ([vp, vp, i64, vp, vp, vp, i32, i32, vp, ip], i32),
        "tp_chunk_copy_ex": ([vp, vp, i64, i32, vp, vp, vp, i32, i32, vp, ip], i32),
        "tp_plan_row_shift": ([vp, vp, i64, i64, pp], i32),
        "tp_plan_pipelined_map": ([vp, vp, i64, i32, i32, i32, i32, i32, i32, i32, i64, pp], i32),
        "tp_plan_chunk_copy": ([vp, vp, i64, i32, vp, vp, vp, i32, i32, i64, pp], i32),
        "tp_map_2d": ([vp, i64, vp, i64, i64, i64, i32, i32, i32, i32, i32, i32, vp, ip], i32),
        "tp_plan_map_2d": ([vp, i64, vp, i64, i64, i64, i32, i32, i32, i32, i32, i32, i64, pp],
                           i32),
        "tp_workgroup_copy": ([vp, vp, i64, vp, i64, vp, i32, vp], i32),
        "tp_workgroup_copy_workspace_bytes": ([i64], i64),
        "tp_plan_workgroup_copy": ([vp, vp, i64, vp, i64, vp, i32, pp], i32),
        "tp_workgroup_copy_noalloc": ([vp, vp, i64, vp, i32, vp], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != 0:
        lib = _load()
        raise TilepipeError(status, where, lib.tp_last_hip_error() if status == 6 else 0)


def _stream_handle(tensor, stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(tensor.device)
    return ctypes.c_void_p(stream.cuda_stream)


def _require(t, dtype, what: str):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{what} must be a GPU tensor (libtilepipe has no CPU path)")
    if t.dtype != dtype:
        raise TypeError(f"{what} must have dtype {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")


def _same_device(*ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError(f"tensors on different devices: {devs}")


# ------------------------------------------------------------------ calls
def device_check(device: int = 0) -> None:
    """Raise TilepipeError unless `device` is a gfx950 GPU."""
    _check(_load().tp_device_check(device), "tp_device_check")


def lds_budget(device: int = 0) -> int:
    """Bytes of LDS one workgroup may use on `device`."""
    v = ctypes.c_int64(0)
    _check(_load().tp_device_lds_budget(device, ctypes.byref(v)), "tp_device_lds_budget")
    return v.value


def row_shift(a, b=None, stream=None) -> Path:
    """b[i, :] = a[(i + 1) % rows, :] for (rows, 4) float32 GPU tensors."""
    import torch
    _require(a, torch.float32, "a")
    if a.dim() != 2 or a.shape[1] != 4:
        raise ValueError("a must have shape (rows, 4)")
    if b is None:
        b = torch.empty_like(a)
    _require(b, torch.float32, "b")
    if b.shape != a.shape:
        raise ValueError("b must have the shape of a")
    _same_device(a, b)
    path = ctypes.c_int(0)
    with torch.cuda.device(a.device):
        st = _load().tp_row_shift(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr()),
                                  a.shape[0], _stream_handle(a, stream), ctypes.byref(path))
    _check(st, "tp_row_shift")
    return Path(path.value)


def pipelined_map(x, y=None, op: str = "scale2", tile_elems: int = 1024, stages: int = 2,
                  tiles_per_block: int = 0, stream=None, resident_cap: int = 0,
                  schedule: "Schedule | str" = "uniform",
                  align: "Align | str" = "realign") -> Path:
    """y[i] = op(x[i]) for float32 GPU tensors (any shape, contiguous).

    Each workgroup streams tiles_per_block consecutive tiles (0: the
    library default, 4 for tiles of at most 512 floats, else 2). resident_cap bounds the workgroups per CU
    (0: the library's policy, -1: no bound, k: about k). schedule "uniform"
    (every wave loads its own part) or "role_split" (one wave loads, the
    others compute). align "realign" (16-byte accesses at any 4-byte
    alignment, stores aligned to y) or "words" (4-byte words on a side that
    is not 16-byte aligned)."""
    import torch
    if op not in OPS:
        raise ValueError(f"unknown op {op!r}; expected one of {sorted(OPS)}")
    _require(x, torch.float32, "x")
    if y is None:
        y = torch.empty_like(x)
    _require(y, torch.float32, "y")
    if y.numel() != x.numel():
        raise ValueError("y must have as many elements as x")
    _same_device(x, y)
    path = ctypes.c_int(0)
    with torch.cuda.device(x.device):
        st = _load().tp_pipelined_map_ex(ctypes.c_void_p(x.data_ptr()),
                                         ctypes.c_void_p(y.data_ptr()), x.numel(), OPS[op],
                                         tile_elems, stages, tiles_per_block, resident_cap,
                                         _schedule(schedule), _align(align),
                                         _stream_handle(x, stream), ctypes.byref(path))
    _check(st, "tp_pipelined_map_ex")
    return Path(path.value)


def _row_stride(t, name: str) -> int:
    """Elements between the rows of a 2-D float32 view with unit column stride."""
    if t.dim() != 2:
        raise ValueError(f"{name} must be a 2-D view")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride")
    return t.stride(0) if t.shape[0] > 1 else max(1, t.shape[1])   # one row: any stride will do


def map_2d(src, dst, op: str = "scale2", box_rows: int = 0, box_cols: int = 0,
           stages: int = 2, boxes_per_block: int = 0, stream=None,
           align: "Align | str" = "realign") -> Path:
    """dst[r, c] = op(src[r, c]) for two same-shape 2-D float32 GPU views with
    unit column stride (rows any number of elements apart). box 0 x 0: the
    library's choice (1024 floats, as wide as the window allows). align as
    for pipelined_map."""
    import torch
    if op not in OPS:
        raise ValueError(f"unknown op {op!r}; expected one of {sorted(OPS)}")
    for t, name in ((src, "src"), (dst, "dst")):
        if t.dtype != torch.float32 or not t.is_cuda:
            raise TypeError(f"{name} must be a float32 CUDA tensor")
    if tuple(src.shape) != tuple(dst.shape):
        raise ValueError("src and dst must have the same shape")
    _same_device(src, dst)
    rows, cols = src.shape
    path = ctypes.c_int(0)
    with torch.cuda.device(src.device):
        st = _load().tp_map_2d(ctypes.c_void_p(src.data_ptr()), _row_stride(src, "src"),
                               ctypes.c_void_p(dst.data_ptr()), _row_stride(dst, "dst"),
                               rows, cols, OPS[op], box_rows, box_cols, stages, boxes_per_block,
                               _align(align), _stream_handle(src, stream), ctypes.byref(path))
    _check(st, "tp_map_2d")
    return Path(path.value)


def chunk_copy(src, dst, pred=None, src_size=None, ignore_src=None, stages: int = 2,
               tiles_per_block: int = 0, stream=None, chunk_bytes: int = 16) -> Path:
    """Predicated copy of chunks of chunk_bytes (4, 8 or 16) bytes: src/dst are
    uint8 GPU tensors of n_chunks*chunk_bytes bytes; pred/src_size/ignore_src
    uint8 tensors of n_chunks (or None)."""
    import torch
    _require(src, torch.uint8, "src")
    _require(dst, torch.uint8, "dst")
    if chunk_bytes not in (4, 8, 16):
        raise ValueError("chunk_bytes must be 4, 8 or 16")
    if src.numel() != dst.numel() or src.numel() % chunk_bytes:
        raise ValueError(f"src and dst must hold the same whole number of {chunk_bytes}-byte chunks")
    n = src.numel() // chunk_bytes
    ptrs = []
    for name, m in (("pred", pred), ("src_size", src_size), ("ignore_src", ignore_src)):
        if m is None:
            ptrs.append(None)
            continue
        _require(m, torch.uint8, name)
        if m.numel() != n:
            raise ValueError(f"{name} must have one byte per chunk")
        ptrs.append(ctypes.c_void_p(m.data_ptr()))
    _same_device(src, dst, pred, src_size, ignore_src)
    path = ctypes.c_int(0)
    with torch.cuda.device(src.device):
        st = _load().tp_chunk_copy_ex(ctypes.c_void_p(src.data_ptr()),
                                      ctypes.c_void_p(dst.data_ptr()), n, chunk_bytes, *ptrs,
                                      stages, tiles_per_block, _stream_handle(src, stream),
                                      ctypes.byref(path))
    _check(st, "tp_chunk_copy_ex")
    return Path(path.value)


def workgroup_copy_workspace_bytes(n_chunks: int) -> int:
    """Bytes of workspace a copy between n_chunks workgroups needs."""
    v = _load().tp_workgroup_copy_workspace_bytes(n_chunks)
    if v < 0:
        raise ValueError("n_chunks out of range")
    return v


def workgroup_copy(src, dst, workspace=None, status=None, spin_limit: int = 0, stream=None):
    """Copies between workgroups: chunk k of dst (256 bytes) receives chunk
    k - 1 of src, handed from workgroup k - 1 to workgroup k; dst chunk 0 is
    not written. src, dst: uint8 GPU tensors of the same whole number of
    256-byte chunks. workspace: uint8 GPU tensor of at least
    workgroup_copy_workspace_bytes(n) bytes, 8-byte aligned (allocated here
    when None).
    status: int32 GPU tensor of one element (allocated when None), 0 after the
    stream has run the call, 1 if some receiver gave up waiting. Returns the
    status tensor (reading it synchronizes)."""
    import torch
    _require(src, torch.uint8, "src")
    _require(dst, torch.uint8, "dst")
    if src.numel() != dst.numel() or src.numel() % 256:
        raise ValueError("src and dst must hold the same whole number of 256-byte chunks")
    n = src.numel() // 256
    if workspace is None:
        workspace = torch.empty(max(1, workgroup_copy_workspace_bytes(n)), dtype=torch.uint8,
                                device=src.device)
    if status is None:
        status = torch.empty(1, dtype=torch.int32, device=src.device)
    _require(workspace, torch.uint8, "workspace")
    _require(status, torch.int32, "status")
    _same_device(src, dst, workspace, status)
    with torch.cuda.device(src.device):
        st = _load().tp_workgroup_copy(ctypes.c_void_p(src.data_ptr()),
                                       ctypes.c_void_p(dst.data_ptr()), n,
                                       ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                                       ctypes.c_void_p(status.data_ptr()), spin_limit,
                                       _stream_handle(src, stream))
    _check(st, "tp_workgroup_copy")
    return status


def workgroup_copy_noalloc(src, dst, status, spin_limit: int = 0, stream=None):
    """workgroup_copy with the library's static per-device workspace (at most
    16384 chunks; calls overlapping on one GPU race). status: int32 GPU
    tensor of one element, written by the call."""
    import torch
    _require(src, torch.uint8, "src")
    _require(dst, torch.uint8, "dst")
    _require(status, torch.int32, "status")
    if src.numel() != dst.numel() or src.numel() % 256:
        raise ValueError("src and dst must hold the same whole number of 256-byte chunks")
    _same_device(src, dst, status)
    with torch.cuda.device(src.device):
        st = _load().tp_workgroup_copy_noalloc(ctypes.c_void_p(src.data_ptr()),
                                               ctypes.c_void_p(dst.data_ptr()), src.numel() // 256,
                                               ctypes.c_void_p(status.data_ptr()), spin_limit,
                                               _stream_handle(src, stream))
    _check(st, "tp_workgroup_copy_noalloc")
    return status


# --------------------------------------------------------- host-only plans
_NO_BUDGET = (1 << 62)


def _plan(status: int, cp: _CPlan, where: str) -> Plan:
    _check(status, where)
    return Plan(Path(cp.path), cp.stages, cp.tile_units, cp.threads, cp.lane_chunks,
                cp.tiles_per_block, cp.lds_bytes, cp.wait_steady, cp.num_tiles, cp.grid,
                cp.ring_bytes, cp.resident_cap, Schedule(cp.schedule), cp.chunk_bytes,
                Align(cp.align), cp.head)


def plan_row_shift(a_ptr: int, b_ptr: int, rows: int, lds_budget: int = _NO_BUDGET) -> Plan:
    cp = _CPlan()
    st = _load().tp_plan_row_shift(ctypes.c_void_p(a_ptr), ctypes.c_void_p(b_ptr), rows,
                                   lds_budget, ctypes.byref(cp))
    return _plan(st, cp, "tp_plan_row_shift")


def plan_map(in_ptr: int, out_ptr: int, n: int, op: str = "scale2", tile_elems: int = 1024,
             stages: int = 2, tiles_per_block: int = 0, lds_budget: int = _NO_BUDGET,
             resident_cap: int = 0, schedule: "Schedule | str" = "uniform",
             align: "Align | str" = "realign") -> Plan:
    cp = _CPlan()
    st = _load().tp_plan_pipelined_map(ctypes.c_void_p(in_ptr), ctypes.c_void_p(out_ptr), n,
                                       OPS.get(op, op if isinstance(op, int) else -1),
                                       tile_elems, stages, tiles_per_block, resident_cap,
                                       _schedule(schedule), _align(align), lds_budget,
                                       ctypes.byref(cp))
    return _plan(st, cp, "tp_plan_pipelined_map")


def plan_map_2d(src_ptr: int, src_stride: int, dst_ptr: int, dst_stride: int, rows: int,
                cols: int, op: str = "scale2", box_rows: int = 0, box_cols: int = 0,
                stages: int = 2, boxes_per_block: int = 0, lds_budget: int = _NO_BUDGET,
                align: "Align | str" = "realign") -> Plan:
    cp = _CPlan()
    st = _load().tp_plan_map_2d(ctypes.c_void_p(src_ptr), src_stride, ctypes.c_void_p(dst_ptr),
                                dst_stride, rows, cols,
                                OPS.get(op, op if isinstance(op, int) else -1), box_rows,
                                box_cols, stages, boxes_per_block, _align(align), lds_budget,
                                ctypes.byref(cp))
    return _plan(st, cp, "tp_plan_map_2d")


def plan_chunk_copy(src_ptr: int, dst_ptr: int, n_chunks: int, pred_ptr: int = 0,
                    size_ptr: int = 0, ignore_ptr: int = 0, stages: int = 2,
                    tiles_per_block: int = 0, lds_budget: int = _NO_BUDGET,
                    chunk_bytes: int = 16) -> Plan:
    cp = _CPlan()
    st = _load().tp_plan_chunk_copy(ctypes.c_void_p(src_ptr), ctypes.c_void_p(dst_ptr), n_chunks,
                                    chunk_bytes, ctypes.c_void_p(pred_ptr or None),
                                    ctypes.c_void_p(size_ptr or None),
                                    ctypes.c_void_p(ignore_ptr or None), stages, tiles_per_block,
                                    lds_budget, ctypes.byref(cp))
    return _plan(st, cp, "tp_plan_chunk_copy")


def plan_workgroup_copy(src_ptr: int, dst_ptr: int, n_chunks: int, workspace_ptr: int,
                        workspace_bytes: int, status_ptr: int, spin_limit: int = 0) -> Plan:
    cp = _CPlan()
    st = _load().tp_plan_workgroup_copy(ctypes.c_void_p(src_ptr), ctypes.c_void_p(dst_ptr),
                                        n_chunks, ctypes.c_void_p(workspace_ptr or None),
                                        workspace_bytes, ctypes.c_void_p(status_ptr or None),
                                        spin_limit, ctypes.byref(cp))
    return _plan(st, cp, "tp_plan_workgroup_copy")
