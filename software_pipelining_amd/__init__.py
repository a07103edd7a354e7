"""libtilepipe: software-pipelined global->LDS tile streaming for MI355X (gfx950).

The compute lives in hand-written HIP kernels inside ``libtilepipe.so`` behind a
C ABI (``include/tilepipe.h``). :mod:`software_pipelining_amd.tilepipe` is the
thin ctypes binding; it loads the library on first use and raises if it has not
been built; there is no CPU fallback.
"""
from .tilepipe import (  # noqa: F401
    Align, TilepipeError, Path, Plan, Schedule, chunk_copy, device_check, lds_budget, library_path,
    map_2d, pipelined_map, plan_chunk_copy, plan_map, plan_map_2d, plan_row_shift,
    plan_workgroup_copy, row_shift, workgroup_copy, workgroup_copy_noalloc,
    workgroup_copy_workspace_bytes,
)

__all__ = [
    "Align", "TilepipeError", "Path", "Plan", "Schedule", "chunk_copy", "device_check", "lds_budget",
    "library_path", "map_2d", "pipelined_map", "plan_chunk_copy", "plan_map", "plan_map_2d",
    "plan_row_shift", "plan_workgroup_copy", "row_shift", "workgroup_copy",
    "workgroup_copy_noalloc", "workgroup_copy_workspace_bytes",
]
