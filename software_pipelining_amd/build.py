"""Build libtilepipe.so for gfx950 (hipcc) in-tree.

    python -m software_pipelining_amd.build [--jobs N]

Translation units compile in parallel into ``_build/`` at the repository root;
the shared library is written next to this file. The planner (tp_plan.cpp) is
plain C++ and is compiled by g++ to keep it free of HIP.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys
import time
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtilepipe.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 (results must stay bit-exact and
# some packed forms are not trusted); IEEE denormals; no FP contraction beyond
# the explicit fmaf calls.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=off",
    "-Wall", "-Wno-unused-command-line-argument",
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wextra", "-Werror"]

# The kernel families are instantiated per op and per half of the stage range
# (one compilation of tp_<family>_inst.hip each), heaviest first, so the
# pieces spread evenly over the compile jobs.
_OPS = (("scale2", "TP_OP_SCALE2"), ("horner32", "TP_OP_HORNER32"), ("copy", "TP_OP_COPY"))
_HALVES = ((1, 4), (5, 8))
INSTANCES = [
    (f"tp_{fam}_inst.hip", f"tp_{fam}_{op}_s{lo}_{hi}",
     [f"-DTP_INST_OP={macro}", f"-DTP_INST_SLO={lo}", f"-DTP_INST_SHI={hi}",
      f"-DTP_INST_FN=launch_{fam}_{op}_s{lo}_{hi}"])
    for fam in ("map2d", "map_split", "map") for lo, hi in reversed(_HALVES) for op, macro in _OPS
]
HIP_SOURCES = ["tp_chunk_copy.hip", "tp_row_shift.hip", "tp_wg_copy.hip", "tp_api.cpp"]
CXX_SOURCES = ["tp_plan.cpp"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr).strip()
    # hipcc's host pass does not know the packed-fp32 target feature: harmless
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + "\n".join(lines))
    return "\n".join(lines)


def _compile(unit, save_temps: bool = False) -> str:
    """unit: a source file name, or (source, object stem, extra flags)."""
    src, stem, defs = (unit, os.path.splitext(unit)[0], []) if isinstance(unit, str) else unit
    obj = os.path.join(BUILD, stem + ".o")
    path = os.path.join(CSRC, src)
    if src in CXX_SOURCES:
        cmd = ["g++", *CXX_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, *HIP_FLAGS, *defs, "-x", "hip", f"-I{INCLUDE}", f"-I{CSRC}", "-c", path,
               "-o", obj]
        if save_temps:
            cmd += ["-save-temps=obj"]
    _run(cmd)
    return obj


def build(jobs: int | None = None, verbose: bool = True, save_temps: bool = False) -> str:
    """Compile every translation unit and link libtilepipe.so; return its path."""
    os.makedirs(BUILD, exist_ok=True)
    t0 = time.time()
    units = INSTANCES + HIP_SOURCES + CXX_SOURCES
    jobs = jobs or min(len(units), max(1, os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda u: _compile(u, save_temps), units))
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print(f"[build] {LIB} ({time.time() - t0:.1f}s)", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--save-temps", action="store_true",
                    help="keep the gfx950 assembly in _build/ for inspection")
    a = ap.parse_args()
    build(a.jobs, save_temps=a.save_temps)
