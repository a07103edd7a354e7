"""CPU emulator of libtilepipe's kernel bodies (test infrastructure only).

``tp_emu.cpp`` compiles the library's own kernel-body templates for the host
against an emulated engine (see its header comment for what it checks) and
links the library's host planner, so a launch is planned and laid out exactly
as the C ABI would launch it. Nothing here is reachable from the library.

The shared library is built into ``_build/emu/`` at the repository root the
first time a test asks for it, or when one of its sources is newer.
"""
from __future__ import annotations

import ctypes
import glob
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "software_pipelining_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(ROOT, "_build", "emu")
LIB = os.path.join(OUT, "libtpemu.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


# (source, EMU_PART): each compilation holds part of the kernel instances
UNITS = [("tp_emu_chunk.cpp", 0), ("tp_emu_map.cpp", 0), ("tp_emu_map.cpp", 1),
         ("tp_emu_map.cpp", 2), ("tp_emu_map2d.cpp", 0), ("tp_emu_map2d.cpp", 1)]


def _sources():
    return ([os.path.join(HERE, f) for f in ("tp_emu.hpp", "tp_emu_chunk.cpp", "tp_emu_map.cpp",
                                             "tp_emu_map2d.cpp")] +
            [os.path.join(CSRC, "tp_plan.cpp"), os.path.join(INCLUDE, "tilepipe.h")] +
            glob.glob(os.path.join(CSRC, "*.hpp")))


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError("emulator build failed: " + " ".join(cmd) + "\n" + r.stderr[-4000:])


def _fresh() -> bool:
    return (os.path.exists(LIB) and
            os.path.getmtime(LIB) >= max(os.path.getmtime(s) for s in _sources()))


def build(force: bool = False) -> str:
    """Compile the emulator (host code only, the compilations in parallel) and
    link it with the library's planner. Test processes running side by side
    (pytest -n) take a file lock, so one builds and the others reuse it."""
    if not force and _fresh():
        return LIB
    import fcntl
    os.makedirs(OUT, exist_ok=True)
    with open(os.path.join(OUT, ".build.lock"), "w") as lock:
        fcntl.flock(lock, fcntl.LOCK_EX)
        if not force and _fresh():
            return LIB
        return _build_locked()


def _build_locked() -> str:
    from concurrent.futures import ThreadPoolExecutor
    inc = [f"-I{INCLUDE}", f"-I{CSRC}"]
    cmds, objs = [], []
    for src, part in UNITS:
        obj = os.path.join(OUT, f"{os.path.splitext(src)[0]}_{part}.o")
        # -O0: the bodies' always-inlined steps compile several times faster,
        # and the fiber switches dominate the run time anyway
        cmds.append([HIPCC, "-x", "hip", "--offload-host-only", "-O0", "-std=c++17", "-fPIC",
                     "-ffp-contract=off", "-Wall", f"-DEMU_PART={part}", *inc, "-c",
                     os.path.join(HERE, src), "-o", obj])
        objs.append(obj)
    plan_o = os.path.join(OUT, "tp_plan.o")
    cmds.append(["g++", "-O2", "-std=c++17", "-fPIC", *inc, "-c",
                 os.path.join(CSRC, "tp_plan.cpp"), "-o", plan_o])
    objs.append(plan_o)
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as ex:
        list(ex.map(_run, cmds))
    _run(["g++", "-shared", "-o", LIB + ".tmp", *objs])
    os.replace(LIB + ".tmp", LIB)
    return LIB


class Region(ctypes.Structure):
    _fields_ = [("lo", ctypes.c_uint64), ("hi", ctypes.c_uint64), ("writable", ctypes.c_int)]


class Options(ctypes.Structure):
    _fields_ = [("policy", ctypes.c_int), ("wait_bias", ctypes.c_int), ("seed", ctypes.c_uint64),
                ("lds_base", ctypes.c_uint32), ("regions", ctypes.POINTER(Region)),
                ("n_regions", ctypes.c_int), ("blocks", ctypes.POINTER(ctypes.c_int64)),
                ("n_blocks", ctypes.c_int), ("oor_fill", ctypes.c_int),
                ("drop_barriers", ctypes.c_int)]


class EmulationError(AssertionError):
    pass


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
    return _lib


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _region(r):
    """(array, writable) -> the array's bytes; (lo, hi, writable) -> [lo, hi)."""
    if len(r) == 3:
        return Region(r[0], r[1], int(r[2]))
    a, w = r
    return Region(a.ctypes.data, a.ctypes.data + a.nbytes, int(w))


def _options(regions, policy, seed, wait_bias, lds_base, blocks):
    regs = (Region * len(regions))(*[_region(r) for r in regions])
    # policy 0/1: loads land at retirement / at issue; + 2: out-of-range lanes
    # leave random bytes in LDS instead of zeros; + 4: barriers do nothing (a
    # planted mistake)
    o = Options(policy & 1, wait_bias, seed, lds_base, regs, len(regions), None, 0,
                (policy >> 1) & 1, (policy >> 2) & 1)
    keep = [regs]
    if blocks is not None:
        arr = (ctypes.c_int64 * len(blocks))(*blocks)
        o.blocks = arr
        o.n_blocks = len(blocks)
        keep.append(arr)
    return o, keep


VIOLATION, NOT_INSTANTIATED = -1, -2


def _call(name, args, regions, policy, seed, wait_bias, lds_base, blocks):
    o, keep = _options(regions, policy, seed, wait_bias, lds_base, blocks)
    from software_pipelining_amd.tilepipe import _CPlan  # the ABI's tp_plan struct
    plan = _CPlan()
    err = ctypes.create_string_buffer(1024)
    f = getattr(lib(), name)
    f.restype = ctypes.c_int
    st = f(*args, ctypes.byref(o), ctypes.byref(plan), err, len(err))
    del keep
    if st == VIOLATION:
        raise EmulationError(err.value.decode())
    if st == NOT_INSTANTIATED:
        raise NotImplementedError(f"{name}: this kernel instance is not compiled into the emulator")
    if st != 0:
        raise ValueError(f"{name}: planning failed with status {st}")
    return plan


def chunk_copy(src, dst, pred=None, src_size=None, ignore_src=None, *, chunk_bytes=16, stages=2,
               tiles_per_block=0, policy=0, seed=0, wait_bias=0, lds_base=0, blocks=None,
               regions=None):
    """Run the chunk copy's kernel body under the emulator on host numpy
    buffers. `regions` (default: the five arrays of the call) are the
    (array, writable) pairs an access may touch. Returns the launch plan's
    grid; raises EmulationError on the first violation."""
    n = dst.nbytes // chunk_bytes
    if regions is None:
        regions = [(src, False), (dst, True)] + [(m, False) for m in (pred, src_size, ignore_src)
                                                 if m is not None]
    args = (_ptr(src), _ptr(dst), ctypes.c_int64(n), chunk_bytes, _ptr(pred), _ptr(src_size),
            _ptr(ignore_src), stages, tiles_per_block)
    return _call("emu_chunk_copy", args, regions, policy, seed, wait_bias, lds_base, blocks)


_OPS = {"scale2": 0, "horner32": 1, "copy": 2}
_SCHED = {"uniform": 0, "role_split": 1}
_ALIGN = {"realign": 0, "words": 1}


def pipelined_map(x, y, op="scale2", tile_elems=256, stages=2, tiles_per_block=0, *,
                  resident_cap=0, schedule="uniform", align="realign", policy=0, seed=0,
                  wait_bias=0, lds_base=0, blocks=None, regions=None):
    """The 1-D map's kernel body under the emulator: y = op(x) for float32
    numpy arrays (views at any 4-byte offset)."""
    if regions is None:
        regions = [(x, False), (y, True)] if x.ctypes.data != y.ctypes.data else [(y, True)]
    args = (_ptr(x), _ptr(y), ctypes.c_int64(x.size), _OPS[op], tile_elems, stages, tiles_per_block,
            resident_cap, _SCHED[schedule], _ALIGN[align])
    return _call("emu_pipelined_map", args, regions, policy, seed, wait_bias, lds_base, blocks)


def map_2d(src, dst, op="scale2", box_rows=0, box_cols=0, stages=2, boxes_per_block=0, *,
           align="realign", policy=0, seed=0, wait_bias=0, lds_base=0, blocks=None,
           regions=None, src_region=None, dst_region=None):
    """The 2-D map's kernel body under the emulator: src and dst are 2-D
    float32 views with unit column stride. An access may touch the bytes from
    a view's first element to its last (src_region / dst_region replace
    those, as (lo, hi, writable) or (array, writable))."""
    rows, cols = src.shape
    ss, ds = src.strides[0] // 4, dst.strides[0] // 4
    if regions is None:
        def span(a, w):
            lo = a.ctypes.data
            return (lo, lo + ((a.shape[0] - 1) * a.strides[0] + 4 * a.shape[1] if a.size else 0), w)
        regions = [src_region if src_region is not None else span(src, False),
                   dst_region if dst_region is not None else span(dst, True)]
    args = (_ptr(src), ctypes.c_int64(ss), _ptr(dst), ctypes.c_int64(ds), ctypes.c_int64(rows),
            ctypes.c_int64(cols), _OPS[op], box_rows, box_cols, stages, boxes_per_block,
            _ALIGN[align])
    return _call("emu_map_2d", args, regions, policy, seed, wait_bias, lds_base, blocks)


def row_shift(a, b, *, policy=0, seed=0, wait_bias=0, lds_base=0, regions=None):
    """The row exchange's kernel body under the emulator (float32 rows x 4)."""
    if regions is None:
        regions = [(a, False), (b, True)] if a.ctypes.data != b.ctypes.data else [(b, True)]
    args = (_ptr(a), _ptr(b), ctypes.c_int64(a.shape[0]))
    return _call("emu_row_shift", args, regions, policy, seed, wait_bias, lds_base, None)


def workgroup_copy(src, dst, workspace, status, *, spin_limit=0, policy=0, seed=0, lds_base=0,
                   blocks=None, regions=None):
    """Copies between workgroups under the emulator on host numpy buffers
    (uint8 src/dst/workspace, int32 status of one element). `blocks` orders
    the hand-off kernel's workgroups (default: 0, 1, ...)."""
    n = dst.nbytes // 256
    if regions is None:
        regions = [(src, False), (dst, True), (workspace, True), (status, True)]
        if src.ctypes.data == dst.ctypes.data:
            regions = regions[1:]
    args = (_ptr(src), _ptr(dst), ctypes.c_int64(n), _ptr(workspace),
            ctypes.c_int64(workspace.nbytes), _ptr(status), spin_limit)
    return _call("emu_workgroup_copy", args, regions, policy, seed, 0, lds_base, blocks)
