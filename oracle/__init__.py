"""CPU oracle for libtilepipe — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (the HIP library and its
Python binding) never does and must not: it has no CPU fallback.

The arithmetic lives in ``oracle.c`` (plain C, built by gcc with
``-O2 -ffp-contract=off -fno-fast-math``). This module only marshals numpy
arrays into it and, for large inputs, splits the index range over a thread pool
(ctypes releases the GIL during the call, and every C function works on an
independent ``[lo, hi)`` range, so the split cannot change a result).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

GCC_FLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
             "-fPIC", "-shared", "-Wall", "-Wextra", "-Werror"]

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc and return its path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *GCC_FLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    p, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.oracle_row_shift.argtypes = [p, p, i64]
    lib.oracle_row_shift.restype = None
    for name in ("oracle_map_scale2", "oracle_map_copy", "oracle_map_horner32"):
        getattr(lib, name).argtypes = [p, p, i64, i64]
        getattr(lib, name).restype = None
    lib.oracle_horner32_coeffs.argtypes = [p]
    lib.oracle_horner32_coeffs.restype = None
    lib.oracle_horner32_subnormal_steps.argtypes = [p, i64, i64]
    lib.oracle_horner32_subnormal_steps.restype = i64
    lib.oracle_chunk_copy.argtypes = [p, p, p, p, p, i64, i64]
    lib.oracle_chunk_copy.restype = None
    lib.oracle_chunk_copy_w.argtypes = [p, p, ctypes.c_int, p, p, p, i64, i64]
    lib.oracle_chunk_copy_w.restype = None
    lib.oracle_map_2d.argtypes = [p, i64, p, i64, i64, ctypes.c_int, i64, i64]
    lib.oracle_map_2d.restype = None
    lib.oracle_workgroup_copy.argtypes = [p, p, i64, i64]
    lib.oracle_workgroup_copy.restype = None
    _lib = lib
    return lib


def default_threads() -> int:
    """Host threads the oracle uses by default: the cores this process may run on."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _ptr(a: np.ndarray | None) -> int | None:
    return None if a is None else a.ctypes.data


def _ranges(n: int, threads: int, min_block: int = 1 << 16):
    parts = max(1, min(threads, (n + min_block - 1) // min_block))
    step = (n + parts - 1) // parts if parts else 0
    return [(lo, min(n, lo + step)) for lo in range(0, n, step)] if n else []


def _run_ranged(fn, args_prefix, n: int, threads: int):
    rs = _ranges(n, threads)
    if len(rs) <= 1:
        for lo, hi in rs:
            fn(*args_prefix, lo, hi)
        return
    with ThreadPoolExecutor(max_workers=len(rs)) as ex:
        list(ex.map(lambda r: fn(*args_prefix, r[0], r[1]), rs))


def _contig(a: np.ndarray, dtype) -> np.ndarray:
    if a.dtype != dtype:
        raise TypeError(f"expected dtype {dtype}, got {a.dtype}")
    return np.ascontiguousarray(a)


# ---------------------------------------------------------------- row shift
def row_shift(a: np.ndarray) -> np.ndarray:
    """b[i, :] = a[(i + 1) % rows, :] for a (rows, 4) float32 array, bitwise."""
    if a.ndim != 2 or a.shape[1] != 4:
        raise ValueError("row_shift expects a (rows, 4) array")
    a = _contig(a, np.float32)
    b = np.empty_like(a)
    if a.shape[0]:
        _load().oracle_row_shift(_ptr(a), _ptr(b), a.shape[0])
    return b


# ---------------------------------------------------------------------- map
_MAP_FN = {"scale2": "oracle_map_scale2", "horner32": "oracle_map_horner32",
           "copy": "oracle_map_copy"}


def pipelined_map(x: np.ndarray, op: str = "scale2", threads: int | None = None,
                  out: np.ndarray | None = None) -> np.ndarray:
    """out[i] = op(x[i]) on a 1-D float32 array (the plain definition: no tiles)."""
    if op not in _MAP_FN:
        raise ValueError(f"unknown op {op!r}")
    x = _contig(x.reshape(-1), np.float32)
    if out is None:
        out = np.empty_like(x)
    fn = getattr(_load(), _MAP_FN[op])
    _run_ranged(fn, (_ptr(x), _ptr(out)), x.size, threads or default_threads())
    return out


_OP_CODE = {"scale2": 0, "horner32": 1, "copy": 2}


def map_2d(src: np.ndarray, dst: np.ndarray, op: str = "scale2",
           threads: int | None = None) -> np.ndarray:
    """dst[r, c] = op(src[r, c]) for 2-D float32 views with unit column stride
    (rows may lie any number of elements apart); writes into dst in place and
    returns it. Elements of dst's underlying buffer outside the view are not
    touched."""
    if op not in _OP_CODE:
        raise ValueError(f"unknown op {op!r}")
    for a in (src, dst):
        if a.ndim != 2 or a.dtype != np.float32 or (a.shape[1] > 1 and a.strides[1] != 4) \
                or a.strides[0] < 0 or a.strides[0] % 4:
            raise ValueError("map_2d expects 2-D float32 views with unit column stride")
    if src.shape != dst.shape:
        raise ValueError("src and dst must have the same shape")
    rows, cols = src.shape
    if rows == 0 or cols == 0:
        return dst
    lib = _load()
    args = (src.ctypes.data, src.strides[0] // 4, dst.ctypes.data, dst.strides[0] // 4, cols,
            _OP_CODE[op])
    threads = threads or default_threads()
    parts = max(1, min(threads, rows, (rows * cols + (1 << 16) - 1) >> 16))
    step = -(-rows // parts)
    rs = [(lo, min(rows, lo + step)) for lo in range(0, rows, step)]
    if len(rs) == 1:
        lib.oracle_map_2d(*args, 0, rows)
    else:
        with ThreadPoolExecutor(max_workers=len(rs)) as ex:
            list(ex.map(lambda r: lib.oracle_map_2d(*args, r[0], r[1]), rs))
    return dst


def horner32_coeffs() -> np.ndarray:
    c = np.zeros(32, dtype=np.float32)
    _load().oracle_horner32_coeffs(_ptr(c))
    return c


def horner32_subnormal_steps(x: np.ndarray, threads: int | None = None) -> int:
    x = _contig(x.reshape(-1), np.float32)
    rs = _ranges(x.size, threads or default_threads())
    fn = _load().oracle_horner32_subnormal_steps
    with ThreadPoolExecutor(max_workers=max(1, len(rs))) as ex:
        return int(sum(ex.map(lambda r: fn(_ptr(x), r[0], r[1]), rs)))


# --------------------------------------------------------------- chunk copy
def chunk_copy(src: np.ndarray, dst: np.ndarray, pred: np.ndarray | None = None,
               src_size: np.ndarray | None = None, ignore_src: np.ndarray | None = None,
               threads: int | None = None, chunk_bytes: int = 16) -> np.ndarray:
    """Return a new array: dst after the predicated chunk copy.

    src and dst are uint8 arrays of n_chunks * chunk_bytes bytes (any shape),
    chunk_bytes 4, 8 or 16; the metadata arrays are uint8 of n_chunks, or None
    for their defaults.
    """
    if chunk_bytes not in (4, 8, 16):
        raise ValueError("chunk_bytes must be 4, 8 or 16")
    src = _contig(src.reshape(-1), np.uint8)
    res = np.array(dst.reshape(-1), dtype=np.uint8, copy=True)
    if src.size != res.size or src.size % chunk_bytes:
        raise ValueError(f"src and dst must hold the same whole number of {chunk_bytes}-byte chunks")
    n = src.size // chunk_bytes
    meta = []
    for m in (pred, src_size, ignore_src):
        if m is not None:
            m = _contig(m.reshape(-1), np.uint8)
            if m.size != n:
                raise ValueError("metadata arrays need one byte per chunk")
        meta.append(m)
    _run_ranged(_load().oracle_chunk_copy_w,
                (_ptr(src), _ptr(res), chunk_bytes, *(_ptr(m) for m in meta)), n,
                threads or default_threads())
    return res.reshape(dst.shape)


# ------------------------------------------------------- copies between workgroups
WORKGROUP_CHUNK = 256


def workgroup_copy(src: np.ndarray, dst: np.ndarray, threads: int | None = None) -> np.ndarray:
    """Return a new array: dst after every group k >= 1 received chunk k - 1 of
    src (256-byte chunks; dst chunk 0 unchanged). src and dst are uint8 arrays
    of the same whole number of chunks."""
    src = _contig(src.reshape(-1), np.uint8)
    out = _contig(dst.reshape(-1), np.uint8).copy()
    if src.size != out.size or src.size % WORKGROUP_CHUNK:
        raise ValueError("src and dst must hold the same whole number of 256-byte chunks")
    n = src.size // WORKGROUP_CHUNK
    rs = _ranges(n, threads or default_threads(), min_block=1 << 12)
    fn = _load().oracle_workgroup_copy
    with ThreadPoolExecutor(max_workers=max(1, len(rs))) as ex:
        list(ex.map(lambda r: fn(_ptr(src), _ptr(out), r[0], r[1]), rs))
    return out
