"""Benchmark of libtilepipe on one MI355X.

One step = one pass of the pipelined map (scale-by-2) over 2**28 float32
(1 GiB read, 1 GiB written), inputs resident in HBM. Prints ONE JSON line with
the achieved HBM bandwidth, its fraction of the MI355X peak, the roofline of
the dominant kernel, the CPU oracle's throughput on the same workload, and the
other rows of the hot path (stage/tile sweep with the misaligned fallback, the
predicated chunk copy, the compute-heavy map at 1/2/4 stages, the small
double-buffered map, the row exchange).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--stages S] [--tile T]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
FP32_VALU_PEAK_TFLOPS = 78.6   # unpacked v_fma_f32: 256 CU x 128 lanes x 2 FLOP x 2.4 GHz
METRIC = "achieved HBM GB/s (read+write) and % of MI355X peak, pipelined map, 1 GPU"


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--stages", type=int, default=2)
    ap.add_argument("--tile", type=int, default=256)
    ap.add_argument("--tiles-per-block", type=int, default=0,
                    help="consecutive tiles per workgroup (0: the library default)")
    ap.add_argument("--quick", action="store_true", help="headline only: no sweep, no extra rows")
    ap.add_argument("--mode", choices=("bench", "stages", "sweep", "occupancy", "map2d", "align",
                                       "strides", "chunk", "misaligned", "map2d_boxes",
                                       "box_strides", "workgroup_copy"),
                    default="bench",
                    help="stages: only the maps at 1-4 stages; sweep: only the 36-point stage/tile "
                         "sweep (both for hardware-counter passes); occupancy: scale2 bandwidth "
                         "against the bound on resident workgroups per CU; map2d: only the 2-D "
                         "map with its default box (for counter passes); align: scale2 bandwidth "
                         "against the offsets of in and out from a 128-byte line, both policies; "
                         "strides: 2-D map bandwidth against the source's row padding and the "
                         "run width; chunk: only the chunk copy (the points of "
                         "CHUNK_COUNTER_POINTS, in order) and the runtime's 1 GiB copy, for "
                         "counter passes; misaligned: scale2 with the source on or 4 bytes off "
                         "a line against the run length (MISALIGNED_POINTS); map2d_boxes: the "
                         "2-D map with each box of MAP2D_BOXES in order, for counter passes; "
                         "box_strides: those boxes at each row-stride pair of BOX_STRIDE_PAIRS; "
                         "workgroup_copy: the copy between workgroups' row alone")
    ap.add_argument("--rounds", type=int, default=1,
                    help="interleaved rounds of --mode misaligned and --mode box_strides")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU work: read the rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE outputs "
                         "of two runs of `bench.py --quick --no-cpu-baseline` (defaults otherwise), "
                         "scale each counter by what it reads for the runtime's 1 GiB copy, and "
                         "store the step's HBM bytes per launch in profiles/traffic.json")
    ap.add_argument("--record-chunk-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU work: the same for two runs of `bench.py --mode chunk`: store the "
                         "HBM bytes per launch of each point of CHUNK_COUNTER_POINTS")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle baseline")
    return ap.parse_args()


# ------------------------------------------------------------------ timing
def time_launches(fn, warmup: int, steps: int):
    """Run fn warmup times, then `steps` times between events on the current
    stream (the one the library launches on). Returns (per-launch ms list,
    whole-region ms)."""
    import torch
    s = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    r0 = torch.cuda.Event(enable_timing=True)
    r1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    r0.record(s)
    for i in range(steps):
        starts[i].record(s)
        fn()
        ends[i].record(s)
    r1.record(s)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    return per, r0.elapsed_time(r1)


def gpu_warmup(fn, ms: float = 150.0):
    """Keep the GPU busy with fn for about `ms` milliseconds. Coming out of idle
    the clocks take some 20 ms of sustained load to ramp up; launches timed
    before that run up to a fifth slower, whichever configuration comes first."""
    import torch
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    fn()
    e1.record(s)
    torch.cuda.synchronize()
    reps = max(1, int(ms / max(e0.elapsed_time(e1), 1e-3)))
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()


def time_region(fn, warmup: int, steps: int) -> float:
    """Milliseconds for `steps` back-to-back calls after `warmup` untimed ones,
    bracketed by two events on the current stream (no events in between)."""
    import torch
    s = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    r0 = torch.cuda.Event(enable_timing=True)
    r1 = torch.cuda.Event(enable_timing=True)
    r0.record(s)
    for _ in range(steps):
        fn()
    r1.record(s)
    torch.cuda.synchronize()
    return r0.elapsed_time(r1)


def median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


# What builds and launches the map kernel: its sources, the planner that sets
# its launch (grid, LDS, residency), the ABI and the compiler flags.
MAP_KERNEL_SOURCES = ["software_pipelining_amd/csrc/" + f for f in (
    "tp_engine.hpp", "tp_internal.hpp", "tp_pipeline.hpp", "tp_map.hpp", "tp_map_inst.hip",
    "tp_plan.cpp", "tp_api.cpp")] + ["include/tilepipe.h", "software_pipelining_amd/build.py"]


# The same for the chunk copy.
CHUNK_KERNEL_SOURCES = ["software_pipelining_amd/csrc/" + f for f in (
    "tp_engine.hpp", "tp_internal.hpp", "tp_chunk_copy.hpp", "tp_chunk_copy.hip", "tp_plan.cpp",
    "tp_api.cpp")] + ["include/tilepipe.h", "software_pipelining_amd/build.py"]


def kernel_source_hash(sources=None) -> str:
    """Hash of what builds and launches a kernel (the map's by default): a stored
    hardware-counter reading is only reported while it still describes the
    kernel being run."""
    h = hashlib.sha256()
    for name in sources or MAP_KERNEL_SOURCES:
        with open(os.path.join(ROOT, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def step_traffic_key(n: int, tile: int, stages: int, tiles_per_block: int) -> str:
    return f"map_scale2_n{n}_t{tile}_s{stages}_T{tiles_per_block}"


def _counter_rows(directory: str, counter: str, with_ids: bool = False):
    """(kernel name, grid size, value) of every dispatch in the rocprofv3
    counter-collection CSVs under `directory` (with_ids: (dispatch id, name,
    grid, value), in dispatch order)."""
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") == counter:
                    rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], int(r["Grid_Size"]),
                                 float(r["Counter_Value"])))
    if not rows:
        raise SystemExit(f"no {counter} rows under {directory}")
    rows.sort()
    return rows if with_ids else [r[1:] for r in rows]


def _copy_calibration_kib(rows):
    """Counter KiB of the runtime's 1 GiB copy: the copyBuffer dispatches with
    the largest grid (it reads and writes exactly 2^30 bytes)."""
    copies = [r for r in rows if "copyBuffer" in r[0]]
    if not copies:
        raise SystemExit("no runtime copy dispatch among the counter rows")
    big = max(g for _, g, _ in copies)
    return median([v for _, g, v in copies if g == big])


def record_traffic(fetch_dir: str, write_dir: str, path: str | None = None):
    """HBM bytes per launch of the step's map kernel from two counter runs.
    Each counter is calibrated on the runtime's device-to-device copy of
    1 GiB that the bench also runs (it reads and writes exactly 2^30 bytes):
    scale = 2^30 / 1 KiB / counter KiB of that copy. The copy's dispatches are
    the copyBuffer ones with the largest grid; the map kernel's value is the
    median over its dispatches."""
    gib_kib = float(1 << 20)
    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(d, counter)
        copy_kib = _copy_calibration_kib(rows)
        maps = [v for k, _, v in rows if "map_kernel<0, 2, 1, true, true>" in k]
        if not maps:
            raise SystemExit(f"no map_kernel<scale2, S=2, L=1, x4, x4> dispatch in {d}")
        out[counter] = {"scale": gib_kib / copy_kib, "map_kib": median(maps), "copy_kib": copy_kib,
                        "dispatches": len(maps)}
    fetch = out["FETCH_SIZE"]["map_kib"] * out["FETCH_SIZE"]["scale"] * 1024
    write = out["WRITE_SIZE"]["map_kib"] * out["WRITE_SIZE"]["scale"] * 1024
    n, tile, stages = 1 << 28, 256, 2
    import software_pipelining_amd as tp
    plan = tp.plan_map(1 << 40, 1 << 41, n, "scale2", tile, stages, 0)   # host-only planning
    key = step_traffic_key(n, tile, stages, plan.tiles_per_block)
    path = path or os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            table = json.load(f)
    except (OSError, ValueError):
        table = {}
    table[key] = {"kernel_source_hash": kernel_source_hash(),
                  "bytes_per_launch": int(round(fetch + write)),
                  "fetch_bytes": int(round(fetch)), "write_bytes": int(round(write)),
                  "scale": {c: round(v["scale"], 5) for c, v in out.items()},
                  "counter_kib": {c: {"map": v["map_kib"], "copy_1GiB": v["copy_kib"],
                                      "map_dispatches": v["dispatches"]} for c, v in out.items()},
                  "source": "profiles/map_scale2_2p28_t256_s2_T4_hbm_traffic.md"}
    with open(path, "w") as f:
        json.dump(table, f, indent=1)
        f.write("\n")
    alg = 8 * n
    log(f"traffic {key}: fetch {fetch:.0f} B, write {write:.0f} B, "
        f"{(fetch + write) / alg:.6f} x the algorithmic {alg} B")


def chunk_traffic_key(operands: str, stages: int, tiles_per_block: int) -> str:
    """Key of a chunk-copy launch over the 2^26-chunk workload, by the ring and
    run the planner chose."""
    return f"chunk_copy_n67108864_{operands}_s{stages}_T{tiles_per_block}"


def record_chunk_traffic(fetch_dir: str, write_dir: str, path: str | None = None):
    """HBM bytes per launch of each point of CHUNK_COUNTER_POINTS from two runs
    of `--mode chunk`: the chunk-copy dispatches, in dispatch order, fall in
    one group per point (one untimed launch, then the timed ones); each
    counter is the median over a group's timed launches, calibrated on the
    runtime's 1 GiB copy as for the map."""
    import software_pipelining_amd as tp
    per = {}
    scale = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(d, counter, with_ids=True)
        scale[counter] = float(1 << 20) / _copy_calibration_kib([r[1:] for r in rows])
        chunk = [v for _, name, _, v in rows if "chunk_copy_kernel" in name]
        k = len(CHUNK_COUNTER_POINTS)
        if not chunk or len(chunk) % k:
            raise SystemExit(f"{len(chunk)} chunk-copy dispatches in {d}: not {k} equal groups")
        g = len(chunk) // k
        for i in range(k):
            per.setdefault(i, {})[counter] = median(chunk[i * g + 1:(i + 1) * g]) * scale[counter] * 1024
    path = path or os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            table = json.load(f)
    except (OSError, ValueError):
        table = {}
    nc = 1 << 26
    for i, (operands, stages, tpb) in enumerate(CHUNK_COUNTER_POINTS):
        plan = tp.plan_chunk_copy(1 << 40, 1 << 41, nc, stages=stages, tiles_per_block=tpb)
        key = chunk_traffic_key(operands, plan.stages, plan.tiles_per_block)
        f, w = per[i]["FETCH_SIZE"], per[i]["WRITE_SIZE"]
        table[key] = {"kernel_source_hash": kernel_source_hash(CHUNK_KERNEL_SOURCES),
                      "bytes_per_launch": int(round(f + w)), "fetch_bytes": int(round(f)),
                      "write_bytes": int(round(w)),
                      "scale": {c: round(v, 5) for c, v in scale.items()},
                      "source": "profiles/chunk_copy_2p26_hbm_traffic.md"}
        log(f"traffic {key}: fetch {f / nc:.3f} B/chunk, write {w / nc:.3f} B/chunk")
    with open(path, "w") as fh:
        json.dump(table, fh, indent=1)
        fh.write("\n")


def stored_traffic(key: str, path: str | None = None, sources=None):
    path = path or os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    e = d.get(key)
    if not e or e.get("kernel_source_hash") != kernel_source_hash(sources):
        return None
    return e.get("bytes_per_launch")


# -------------------------------------------------------------- workloads
def sampled_parity(x_host, y_dev, op, windows=16, width=4096, seed=0):
    """Compare random windows of the GPU output with the oracle on the same
    host input (bitwise)."""
    import numpy as np
    import oracle
    n = x_host.numel()
    rng = np.random.default_rng(seed)
    xs = x_host.numpy()
    for lo in rng.integers(0, max(1, n - width), size=windows):
        hi = min(n, int(lo) + width)
        exp = oracle.pipelined_map(xs[lo:hi], op, threads=1)
        got = y_dev[lo:hi].cpu().numpy()
        if not np.array_equal(got.view(np.uint32), exp.view(np.uint32)):
            return False
    # the start and the ragged end too
    for lo, hi in ((0, min(n, 1000)), (max(0, n - 1000), n)):
        exp = oracle.pipelined_map(xs[lo:hi], op, threads=1)
        if not np.array_equal(y_dev[lo:hi].cpu().numpy().view(np.uint32), exp.view(np.uint32)):
            return False
    return True


def cpu_baseline(x_host, op, bytes_per_elem, seconds):
    """The oracle (untuned) on this host's cores over the same input: whole
    passes over the step's input for about `seconds` of wall time."""
    import oracle
    threads = oracle.default_threads()
    xs = x_host.numpy()
    out = xs.copy()
    times = []
    t_end = time.perf_counter() + seconds
    while True:
        t0 = time.perf_counter()
        oracle.pipelined_map(xs, op, threads=threads, out=out)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() >= t_end:
            break
    t = median(times)
    return {"value": round(bytes_per_elem * xs.size / t / 1e9, 3), "unit": "GB/s",
            "cores": threads, "kind": "oracle",
            "sample": f"the step's full input ({xs.size} floats), {len(times)} passes in "
                      f"{sum(times):.1f} s, median pass {t * 1e3:.1f} ms"}


# Points of the stage counter passes, in launch order: (op, tiles per
# workgroup, bound on resident workgroups per CU, stages), all at tile 1024.
# horner32 at the library's launch (runs of 2, no bound: it fills every wave
# slot), then both ops at 16 tiles per workgroup with no bound (8 workgroups
# per CU, wave-limited), then horner32 at 8 tiles per workgroup and 2
# workgroups per CU (8 waves per CU), then scale2 at the library's launch.
STAGE_COUNTER_POINTS = ([("horner32", 0, 0, S) for S in (1, 2, 4)]
                        + [(op, 16, -1, S) for op in ("horner32", "scale2") for S in (1, 2, 3, 4)]
                        + [("horner32", 8, 2, S) for S in (1, 2, 3, 4)]
                        + [("scale2", 0, 0, S) for S in (1, 2, 4)])


def stages_mode(args):
    """Each point of STAGE_COUNTER_POINTS `steps` times after one untimed
    launch, in that order (a counter pass tells the points apart by dispatch
    order: no other map launch happens in this mode), then the runtime's
    1 GiB copy three times (the traffic counters' calibration)."""
    import torch
    import software_pipelining_amd as tp
    from software_pipelining_amd import workloads
    dev = torch.device("cuda:0")
    xs = {"horner32": workloads.uniform_pm1(1 << 27, seed=4).to(dev),
          "scale2": workloads.uniform_pm1(1 << 28, seed=2).to(dev)}
    ys = {op: torch.empty_like(x) for op, x in xs.items()}
    flat = torch.empty(1 << 28, device=dev)
    # Clocks up under the compute-heavy load the first points run (after a
    # memory-bound warm-up the first horner32 launches ran up to 15 % slower),
    # with the role-split kernel, which is not a map_kernel dispatch.
    gpu_warmup(lambda: tp.pipelined_map(xs["horner32"], ys["horner32"], "horner32", 1024, 2, 0,
                                        schedule="role_split"), 300)
    for op, tpb, cap, S in STAGE_COUNTER_POINTS:
        x, y = xs[op], ys[op]
        f = lambda: tp.pipelined_map(x, y, op, 1024, S, tpb, resident_cap=cap)
        per, _ = time_launches(f, 1, args.steps)
        occ = {0: "library", -1: "8 WG/CU"}.get(cap, f"{cap} WG/CU")
        log(f"{op} tile 1024 T{tpb or 'default'} {occ} S{S}: {median(per) * 1e3:.1f} us")
    out = torch.empty_like(flat)
    for _ in range(3):                           # the traffic counters' calibration
        out.copy_(flat)
    torch.cuda.synchronize()


def sweep_points():
    """The stage/tile sweep of scale-by-2 over 2^28 floats: tile 256/1024/4096 x
    stages 1-4 at the library's run length, with the source 16-byte aligned,
    and at a 4-byte offset both with 16-byte loads (the library's default) and
    with the pages' 4-byte fallback. Consecutive points never launch the same
    kernel on the same grid, so counter passes can tell them apart by order."""
    return ([(0, "realign", T, S) for T in (256, 1024, 4096) for S in (1, 2, 3, 4)] +
            [(1, a, T, S) for a in ("realign", "words") for T in (256, 1024, 4096)
             for S in (1, 2, 3, 4)])


def sweep_mode(args):
    """Each sweep point `steps` times in order, for per-point counter passes
    (a point is told apart by kernel name, grid and workgroup size)."""
    import torch
    import software_pipelining_amd as tp
    from software_pipelining_amd import workloads
    dev = torch.device("cuda:0")
    n = 1 << 28
    xbuf = torch.zeros(n + 4, dtype=torch.float32, device=dev)
    xbuf[:n].copy_(workloads.uniform_pm1(n, seed=2))
    y = torch.empty(n, dtype=torch.float32, device=dev)
    gpu_warmup(lambda: tp.pipelined_map(xbuf[:n], y, "scale2", 256, 2, 0))
    for off, align, T, S in sweep_points():
        xin = xbuf[off:off + n]
        plan = tp.plan_map(xin.data_ptr(), y.data_ptr(), n, "scale2", T, S, 0, align=align)
        per, _ = time_launches(lambda: tp.pipelined_map(xin, y, "scale2", T, S, 0, align=align), 1,
                               args.steps)
        log(f"sweep offset {4 * off}B {align} tile {T} S{S} grid {plan.grid} threads {plan.threads} "
            f"path {tp.Path(plan.path).name.lower()}: {median(per) * 1e3:.1f} us")
    torch.cuda.synchronize()


def map2d_mode(args):
    """The 2-D map workload with the library's default box, `steps` times, plus
    the runtime's 1 GiB copy for the traffic counters' calibration."""
    import torch
    import software_pipelining_amd as tp
    dev = torch.device("cuda:0")
    R, C, SS = MAP2D_ROWS, MAP2D_COLS, MAP2D_SRC_STRIDE
    src = torch.empty(R, SS, device=dev).uniform_(-1, 1)[:, :C]
    dst = torch.empty(R, C, device=dev)
    f = lambda: tp.map_2d(src, dst, "scale2")
    gpu_warmup(f)
    per, _ = time_launches(f, 1, args.steps)
    log(f"map_2d {R}x{C} (row stride {SS}), default box: {median(per) * 1e3:.1f} us, "
        f"{8 * R * C / (median(per) * 1e-3) / 1e9:.0f} GB/s")
    flat = torch.empty(1 << 28, device=dev)
    out = torch.empty_like(flat)
    for _ in range(3):
        out.copy_(flat)
    torch.cuda.synchronize()


def map2d_boxes_mode(args):
    """The 2-D map workload (16384 x 16384 window, row stride 16448) with each
    box of MAP2D_BOXES, `steps` launches each after one untimed, in that order
    (a counter pass tells the boxes apart by dispatch order), then the
    runtime's 1 GiB copy three times (the traffic counters' calibration)."""
    import torch
    import software_pipelining_amd as tp
    dev = torch.device("cuda:0")
    R, C, SS = MAP2D_ROWS, MAP2D_COLS, MAP2D_SRC_STRIDE
    src = torch.empty(R, SS, device=dev).uniform_(-1, 1)[:, :C]
    dst = torch.empty(R, C, device=dev)
    flat = torch.empty(1 << 28, device=dev)
    out = torch.empty_like(flat)
    gpu_warmup(lambda: out.copy_(flat))          # clocks up, no map dispatch
    for br, bc in MAP2D_BOXES:
        f = lambda: tp.map_2d(src, dst, "scale2", br, bc, 2, 0)
        per, _ = time_launches(f, 1, args.steps)
        log(f"map_2d box {br}x{bc}: {median(per) * 1e3:.1f} us, "
            f"{8 * R * C / (median(per) * 1e-3) / 1e9:.0f} GB/s")
    for _ in range(3):
        out.copy_(flat)
    torch.cuda.synchronize()


# (source row stride, destination row stride) pairs of the box-shape comparison,
# in floats: the 2-D workload's own pair first, then both dense, each side alone
# at 64 KiB + 256 B, and both at 64 KiB + 1 KiB.
BOX_STRIDE_PAIRS = [(16448, 16384), (16384, 16384), (16384, 16448), (16448, 16448), (16640, 16640)]


def box_strides_mode(args):
    """scale2 over a 16384 x 16384 window with each box of MAP2D_BOXES (2 stages,
    the library's run), for each row-stride pair of BOX_STRIDE_PAIRS, in
    `rounds` interleaved rounds of `steps` launches; median microseconds."""
    import torch
    import software_pipelining_amd as tp
    dev = torch.device("cuda:0")
    R = C = 16384
    src = {ss: torch.empty(R, ss, device=dev).uniform_(-1, 1)[:, :C]
           for ss in sorted({ss for ss, _ in BOX_STRIDE_PAIRS})}
    gpu_warmup(lambda: tp.map_2d(src[16384], src[16448], "scale2", 1, 1024, 2, 0))
    res = {}
    for _ in range(args.rounds):
        for ss, ds in BOX_STRIDE_PAIRS:
            dst = torch.empty(R, ds, device=dev)[:, :C]
            for br, bc in MAP2D_BOXES:
                f = lambda: tp.map_2d(src[ss], dst, "scale2", br, bc, 2, 0)
                per, _ = time_launches(f, 1, args.steps)
                res.setdefault((ss, ds, br, bc), []).append(median(per) * 1e3)
            del dst
    for ss, ds in BOX_STRIDE_PAIRS:
        log(f"box strides src {ss} dst {ds}: " + "  ".join(
            f"{br}x{bc} {median(res[(ss, ds, br, bc)]):.0f} us" for br, bc in MAP2D_BOXES))
    torch.cuda.synchronize()


def occupancy_mode(args):
    """scale2 over 2^28 at tiles 256/1024/4096, runs of 2/4/8, 1/2/4 stages:
    bandwidth with no bound on resident workgroups, with the library's bound,
    and with every explicit bound, in interleaved rounds."""
    import torch
    import software_pipelining_amd as tp
    dev = torch.device("cuda:0")
    n = 1 << 28
    x = torch.empty(n, device=dev).uniform_(-1, 1)
    y = torch.empty_like(x)
    gpu_warmup(lambda: tp.pipelined_map(x, y, "scale2", 256, 2, 0), 300)
    points = []
    for tile in (256, 1024, 4096):
        waves = min(256, tile // 4) // 64
        for T in (2, 4, 8):
            for S in (1, 2, 4):
                for cap in [-1, 0] + list(range(max(1, 8 // waves), 32 // waves)):
                    points.append((tile, T, S, cap))
    res = {p: [] for p in points}
    for _ in range(2):
        for tile, T, S, cap in points:
            f = lambda: tp.pipelined_map(x, y, "scale2", tile, S, T, resident_cap=cap)
            res[(tile, T, S, cap)].append(8 * n / (time_region(f, 2, args.steps) / args.steps * 1e-3) / 1e9)
    for tile in (256, 1024, 4096):
        for T in (2, 4, 8):
            for S in (1, 2, 4):
                row = {cap: round(median(v)) for (t, tt, s, cap), v in res.items()
                       if (t, tt, s) == (tile, T, S)}
                policy = tp.plan_map(x.data_ptr(), y.data_ptr(), n, "scale2", tile, S, T).resident_cap
                best = max((v, c) for c, v in row.items() if c > 0)
                log(f"occupancy tile {tile} T{T} S{S}: none {row[-1]} policy(cap {policy or '-'}) "
                    f"{row[0]} best cap {best[1]} {best[0]} | " +
                    " ".join(f"{c}:{v}" for c, v in row.items() if c > 0))
    torch.cuda.synchronize()


def chunk_copy_algorithmic_bytes(pred, src_size, ignore_src) -> int:
    """Bytes the predicated copy must move: the three metadata bytes of every
    chunk, the source bytes a written chunk keeps (min(src_size, 16) unless
    ignore_src) and the 16 bytes written for every chunk whose pred is set."""
    import numpy as np
    p = pred.numpy() != 0
    keep = np.minimum(src_size.numpy().astype(np.int64), 16) * (ignore_src.numpy() == 0)
    return int(3 * p.size + (keep * p).sum() + 16 * p.sum())


# Launches of the chunk-copy row: (stages, tiles per workgroup; 0 = the
# library's default run of max(1, S-1) tiles).
CHUNK_ROW_POINTS = [(1, 0), (2, 0), (3, 0), (4, 0), (2, 2), (2, 8), (2, 64)]


def chunk_copy_row(tp, workloads, torch, np, dev, cpu_seconds):
    """The predicated chunk copy over 2^26 chunks: GB/s on the exact
    algorithmic bytes of this instance at every point of CHUNK_ROW_POINTS
    (interleaved rounds), with bit-exact parity of the whole destination
    against the oracle at each; the same instance with every pred set (no
    partly written destination block); 4- and 8-byte chunks; the roofline of
    the default launch; the oracle on the host cores."""
    import oracle
    nc = 1 << 26
    inp = workloads.chunk_copy_inputs(nc, seed=3)
    alg = chunk_copy_algorithmic_bytes(inp.pred, inp.src_size, inp.ignore_src)
    exp = oracle.chunk_copy(inp.src.numpy(), inp.dst_init.numpy(), inp.pred.numpy(),
                            inp.src_size.numpy(), inp.ignore_src.numpy())
    exp_d = torch.from_numpy(exp.reshape(-1)).to(dev)
    del exp
    src = inp.src.reshape(-1).to(dev)
    dst = inp.dst_init.reshape(-1).to(dev)
    meta = [m.to(dev) for m in (inp.pred, inp.src_size, inp.ignore_src)]
    out = {"n_chunks": nc, "algorithmic_bytes": alg, "bytes_per_chunk": round(alg / nc, 3),
           "workload": "2^26 16-byte chunks, pred ~ B(0.9), src_size uniform on {0,4,8,12,16}, "
                       "ignore_src ~ B(0.01), destination pre-filled with 0xDEADBEEF"}
    launch = {}
    parity = True
    for stages, tpb in CHUNK_ROW_POINTS:
        dst.copy_(inp.dst_init.reshape(-1))
        tp.chunk_copy(src, dst, *meta, stages=stages, tiles_per_block=tpb)
        torch.cuda.synchronize()
        parity &= bool(torch.equal(dst, exp_d))   # the copy is idempotent: re-running it
        launch[(stages, tpb)] = []                # rewrites the same bytes
    gpu_warmup(lambda: tp.chunk_copy(src, dst, *meta, stages=2))
    for _ in range(3):
        for stages, tpb in CHUNK_ROW_POINTS:
            per, _ = time_launches(lambda: tp.chunk_copy(src, dst, *meta, stages=stages,
                                                         tiles_per_block=tpb), 1, 6)
            launch[(stages, tpb)] += per
    for stages, tpb in CHUNK_ROW_POINTS:
        plan = tp.plan_chunk_copy(src.data_ptr(), dst.data_ptr(), nc, stages=stages,
                                  tiles_per_block=tpb)
        us = median(launch[(stages, tpb)]) * 1e3
        key = f"S{stages}" + (f"_T{tpb}" if tpb else "_Tdefault")
        out[key] = {"us": round(us, 1), "GBs": round(alg / (us * 1e-6) / 1e9, 1),
                    "pct_peak": round(100 * alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 1),
                    "ring_stages": plan.stages, "tiles_per_block": plan.tiles_per_block}
    out["parity"] = parity
    del exp_d
    # the default launch (2 stages requested, runs of one tile) with every pred set
    ones = torch.ones(nc, dtype=torch.uint8, device=dev)
    per, _ = time_launches(lambda: tp.chunk_copy(src, dst, ones, meta[1], meta[2], stages=2), 2, 10)
    out["pred_all_true_S2_Tdefault_us"] = round(median(per) * 1e3, 1)
    # roofline of the default launch: the algorithmic bytes over its mean
    # per-launch duration; HBM bytes from the counter runs while they still
    # describe this kernel
    dflt = tp.plan_chunk_copy(src.data_ptr(), dst.data_ptr(), nc, stages=2)
    per, _ = time_launches(lambda: tp.chunk_copy(src, dst, *meta, stages=2), 2, 20)
    avg = sum(per) / len(per)
    achieved = alg / (avg * 1e-3) / 1e9
    out["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                       "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                       "traffic": stored_traffic(chunk_traffic_key("workload", dflt.stages,
                                                                   dflt.tiles_per_block),
                                                 sources=CHUNK_KERNEL_SOURCES),
                       "kernel": f"chunk_copy_kernel<{dflt.stages}, 16, x4, x4>",
                       "algorithmic_bytes_per_launch": alg, "avg_launch_us": round(avg * 1e3, 2)}
    # 4- and 8-byte chunks: the same operand arrays over 2^26 chunks of W bytes
    p_ = inp.pred.numpy() != 0
    ign0 = inp.ignore_src.numpy() == 0
    for w in (4, 8):
        algw = int(3 * nc + (np.minimum(inp.src_size.numpy().astype(np.int64), w) * ign0 * p_).sum()
                   + w * p_.sum())
        sw, dw = src[:nc * w], dst[:nc * w]
        row = {"algorithmic_bytes": algw}
        for stages in (2, 3):
            dw.copy_(inp.dst_init.reshape(-1)[:nc * w])
            tp.chunk_copy(sw, dw, *meta, stages=stages, chunk_bytes=w)
            expw = oracle.chunk_copy(inp.src.reshape(-1)[:nc * w].numpy(),
                                     inp.dst_init.reshape(-1)[:nc * w].numpy(),
                                     *(m.numpy() for m in (inp.pred, inp.src_size, inp.ignore_src)),
                                     chunk_bytes=w)
            ok = bool(torch.equal(dw.cpu(), torch.from_numpy(expw.reshape(-1))))
            per, _ = time_launches(lambda: tp.chunk_copy(sw, dw, *meta, stages=stages, chunk_bytes=w),
                                   2, 10)
            us = median(per) * 1e3
            row[f"S{stages}_Tdefault"] = {"us": round(us, 1), "GBs": round(algw / (us * 1e-6) / 1e9, 1),
                                          "parity": ok}
        out[f"width{w}"] = row
    log(f"chunk_copy: {out}")
    out["cpu_baseline"] = chunk_cpu_baseline(inp, min(cpu_seconds, 10.0))
    return out


def workgroup_copy_row(tp, torch, np, dev):
    """Copies between workgroups over 2^20 chunks of 256 bytes (256 MiB): each
    of 2^20 one-wave workgroups hands its chunk to the next through a staging
    slot of tagged 8-byte words. GB/s on the algorithmic bytes (each handed
    chunk read once and written once, 512 B per chunk) and on the 2 KiB each
    chunk moves (source 256, the slot's 512 cleared, 512 stored and at least
    512 loaded, destination 256). Parity of the whole destination against the
    definition."""
    n = 1 << 20
    g = torch.Generator().manual_seed(10)
    src = torch.randint(0, 256, (n * 256,), generator=g, dtype=torch.uint8).to(dev)
    dst = torch.zeros_like(src)
    ws = torch.empty(tp.workgroup_copy_workspace_bytes(n), dtype=torch.uint8, device=dev)
    status = torch.empty(1, dtype=torch.int32, device=dev)
    f = lambda: tp.workgroup_copy(src, dst, ws, status)
    f()
    torch.cuda.synchronize()
    ok = int(status.item()) == 0 and bool(torch.equal(dst[256:], src[:-256]))
    gpu_warmup(f)
    per, _ = time_launches(f, 2, 20)
    us = median(per) * 1e3
    alg = 512 * (n - 1)
    moved = 2048 * (n - 1)
    out = {"n_chunks": n, "chunk_bytes": 256, "us_per_call": round(us, 1),
           "GBs_algorithmic": round(alg / (us * 1e-6) / 1e9, 1),
           "GBs_moved": round(moved / (us * 1e-6) / 1e9, 1),
           "status_ok_and_parity": ok,
           "note": "one call = the clearing kernel plus the hand-off kernel; 2 KiB moves per "
                   "chunk (source, slot cleared, stored and loaded, destination), 512 B of it "
                   "algorithmic"}
    log(f"workgroup_copy: {out}")
    return out


def chunk_cpu_baseline(inp, seconds):
    """The oracle's chunk copy (untuned) on the host cores over the same 2^26
    chunks: whole passes for about `seconds`, GB/s on the algorithmic bytes."""
    import oracle
    threads = oracle.default_threads()
    alg = chunk_copy_algorithmic_bytes(inp.pred, inp.src_size, inp.ignore_src)
    args = [inp.src.numpy(), inp.dst_init.numpy(), inp.pred.numpy(), inp.src_size.numpy(),
            inp.ignore_src.numpy()]
    times = []
    t_end = time.perf_counter() + seconds
    while True:
        t0 = time.perf_counter()
        oracle.chunk_copy(*args, threads=threads)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() >= t_end:
            break
    t = median(times)
    return {"value": round(alg / t / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"the full 2^26-chunk instance, {len(times)} passes in {sum(times):.1f} s, "
                      f"median pass {t * 1e3:.1f} ms (each pass also copies the destination's "
                      f"initial bytes into a new array)"}


def strides_mode(args):
    """scale2 over a 16384 x 16384 window of a source whose rows carry 0-8 KiB
    of padding, into a dense destination, with one-row boxes 256-2048 floats
    wide and runs of 1 and 2 boxes (2 stages), in interleaved rounds."""
    import torch
    import software_pipelining_amd as tp
    dev = torch.device("cuda:0")
    R = C = 16384
    pads = [0, 4, 16, 32, 48, 64, 96, 128, 192, 256, 512, 1024, 2048]
    widths = [256, 512, 1024, 2048]
    src = torch.empty(R * (C + max(pads)), device=dev).uniform_(-1, 1)
    dst = torch.empty(R, C, device=dev)
    gpu_warmup(lambda: tp.map_2d(src[:R * C].view(R, C), dst, "scale2", 1, 1024, 2, 0), 300)
    res = {}
    for _ in range(2):
        for pad in pads:
            s = src[:R * (C + pad)].view(R, C + pad)[:, :C]
            for w in widths:
                for T in (1, 2):
                    f = lambda: tp.map_2d(s, dst, "scale2", 1, w, 2, T)
                    ms = time_region(f, 2, args.steps)
                    res.setdefault((pad, w, T), []).append(8 * R * C / (ms / args.steps * 1e-3) / 1e9)
    for pad in pads:
        log(f"strides pad {pad} floats ({4 * pad} B): " + " ".join(
            f"1x{w} T{T} {median(res[(pad, w, T)]):.0f}" for w in widths for T in (1, 2)))
    torch.cuda.synchronize()


# Points of the chunk-copy counter passes, in launch order: (operands, stages,
# tiles per workgroup). "workload" is the 2^26-chunk instance; "pred_all_true"
# is the same instance with every pred set, so no destination line is left
# partly written.
CHUNK_COUNTER_POINTS = [("workload", 2, 0), ("workload", 3, 0), ("workload", 2, 2),
                        ("workload", 2, 64), ("pred_all_true", 2, 0), ("pred_all_true", 2, 2)]


def chunk_mode(args):
    """The chunk-copy points of CHUNK_COUNTER_POINTS, `steps` launches each after
    one untimed launch, in that order (a counter pass tells them apart by
    dispatch order: no other chunk-copy launch happens in this mode), then the
    runtime's 1 GiB copy three times (the traffic counters' calibration)."""
    import torch
    import software_pipelining_amd as tp
    from software_pipelining_amd import workloads
    dev = torch.device("cuda:0")
    nc = 1 << 26
    inp = workloads.chunk_copy_inputs(nc, seed=3)
    alg = chunk_copy_algorithmic_bytes(inp.pred, inp.src_size, inp.ignore_src)
    src = inp.src.reshape(-1).to(dev)
    dst = inp.dst_init.reshape(-1).to(dev)
    meta = [m.to(dev) for m in (inp.pred, inp.src_size, inp.ignore_src)]
    ones = torch.ones(nc, dtype=torch.uint8, device=dev)
    flat = torch.empty(1 << 28, device=dev)
    out = torch.empty_like(flat)
    gpu_warmup(lambda: out.copy_(flat))          # clocks up, no chunk-copy dispatch
    for operands, stages, tpb in CHUNK_COUNTER_POINTS:
        m = meta if operands == "workload" else [ones, meta[1], meta[2]]
        f = lambda: tp.chunk_copy(src, dst, *m, stages=stages, tiles_per_block=tpb)
        per, _ = time_launches(f, 1, args.steps)
        log(f"chunk copy {operands} S{stages} T{tpb}: {median(per) * 1e3:.1f} us, "
            f"{alg / (median(per) * 1e-3) / 1e9:.0f} GB/s on the workload's {alg} algorithmic bytes")
    for _ in range(3):
        out.copy_(flat)
    torch.cuda.synchronize()


# Points of `--mode misaligned`, in launch order: (source offset in floats,
# tile, tiles per workgroup), scale2 over 2^28 floats at 2 stages.
MISALIGNED_POINTS = [(off, tile, T) for off in (0, 1) for tile in (256, 1024) for T in (2, 3, 4, 8)]


def misaligned_mode(args):
    """scale2 over 2^28 floats with the source on a 256-byte boundary or 4
    bytes past it, tiles 256 and 1024, runs of 2, 3, 4 and 8 tiles, 2 stages
    (the library's residency bound for each): `rounds` interleaved rounds of
    one untimed and `steps` timed launches per point, in the order of
    MISALIGNED_POINTS (with one round, a counter pass tells the points apart by
    dispatch order), then the runtime's 1 GiB copy three times (the traffic
    counters' calibration)."""
    import torch
    import software_pipelining_amd as tp
    dev = torch.device("cuda:0")
    n = 1 << 28
    xb = torch.empty(n + 64, device=dev).uniform_(-1, 1)
    y = torch.empty(n, device=dev)
    if xb.data_ptr() % 256 or y.data_ptr() % 256:
        raise RuntimeError("the buffers must start on a 256-byte boundary")
    flat = torch.empty(1 << 28, device=dev)
    out = torch.empty_like(flat)
    gpu_warmup(lambda: out.copy_(flat))          # clocks up, no map dispatch
    res = {p: [] for p in MISALIGNED_POINTS}
    for _ in range(args.rounds):
        for off, tile, T in MISALIGNED_POINTS:
            x = xb[off:off + n]
            per, _ = time_launches(lambda: tp.pipelined_map(x, y, "scale2", tile, 2, T), 1, args.steps)
            res[(off, tile, T)] += per
    for off, tile, T in MISALIGNED_POINTS:
        us = median(res[(off, tile, T)]) * 1e3
        log(f"misaligned source +{4 * off} B tile {tile} T{T}: {us:.1f} us, "
            f"{8 * n / (us * 1e-6) / 1e9:.0f} GB/s")
    for _ in range(3):
        out.copy_(flat)
    torch.cuda.synchronize()


def align_mode(args):
    """scale2 over 2^28 with in and out at byte offsets from a 256-byte
    boundary, under the library's realignment and under the pages' 4-byte
    fallback, tiles 256 and 1024, 2 stages, in interleaved rounds."""
    import torch
    import software_pipelining_amd as tp
    dev = torch.device("cuda:0")
    n = 1 << 28
    xb = torch.empty(n + 64, device=dev).uniform_(-1, 1)
    yb = torch.empty(n + 64, device=dev)
    if xb.data_ptr() % 256 or yb.data_ptr() % 256:
        raise RuntimeError("the buffers must start on a 256-byte boundary")
    cases = [(0, 0), (16, 16), (64, 64), (0, 16), (0, 64), (0, 128), (4, 0), (16, 0), (64, 0),
             (0, 4), (4, 4), (12, 4)]
    points = [(ci, co, a, t) for ci, co in cases for a in ("realign", "words") for t in (256, 1024)]
    res = {p: [] for p in points}
    gpu_warmup(lambda: tp.pipelined_map(xb[:n], yb[:n], "scale2", 256, 2, 0), 300)
    for _ in range(3):
        for ci, co, a, t in points:
            x, y = xb[ci // 4:ci // 4 + n], yb[co // 4:co // 4 + n]
            f = lambda: tp.pipelined_map(x, y, "scale2", t, 2, 0, align=a)
            per, _ = time_launches(f, 2, args.steps)
            res[(ci, co, a, t)].append(8 * n / (median(per) * 1e-3) / 1e9)
    for ci, co in cases:
        line = []
        for a in ("realign", "words"):
            plan = tp.plan_map(xb.data_ptr() + ci, yb.data_ptr() + co, n, "scale2", 256, 2, 0, align=a)
            gb = " ".join(f"tile {t} {median(res[(ci, co, a, t)]):.0f}" for t in (256, 1024))
            line.append(f"{a} (head {plan.head}, path {tp.Path(plan.path).name.lower()}) {gb}")
        log(f"align in +{ci} B out +{co} B: " + " | ".join(line))
    torch.cuda.synchronize()


def main():
    args = parse()
    if args.record_traffic:
        record_traffic(*args.record_traffic)
        return
    if args.record_chunk_traffic:
        record_chunk_traffic(*args.record_chunk_traffic)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the hot path needs no cross-GPU step and this "
              "build runs on a single MI355X; use --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.mode == "stages":
        stages_mode(args)
        return
    if args.mode == "sweep":
        sweep_mode(args)
        return
    if args.mode == "occupancy":
        occupancy_mode(args)
        return
    if args.mode == "map2d":
        map2d_mode(args)
        return
    if args.mode == "align":
        align_mode(args)
        return
    if args.mode == "strides":
        strides_mode(args)
        return
    if args.mode == "chunk":
        chunk_mode(args)
        return
    if args.mode == "misaligned":
        misaligned_mode(args)
        return
    if args.mode == "map2d_boxes":
        map2d_boxes_mode(args)
        return
    if args.mode == "box_strides":
        box_strides_mode(args)
        return
    if args.mode == "workgroup_copy":
        import numpy as np
        import torch
        import software_pipelining_amd as tp
        print(json.dumps(workgroup_copy_row(tp, torch, np, torch.device("cuda:0"))), flush=True)
        return

    import numpy as np
    import torch

    import software_pipelining_amd as tp
    from software_pipelining_amd import workloads

    dev = torch.device("cuda:0")
    tp.device_check(0)
    props = torch.cuda.get_device_properties(dev)
    log(f"device {props.name} {getattr(props, 'gcnArchName', '')} CUs={props.multi_processor_count} "
        f"LDS/WG={tp.lds_budget(0)}")

    # ---------------------------------------------------------- headline
    n = 1 << 28
    log("generating 2^28 inputs (seed 2)")
    x_host = workloads.uniform_pm1(n, seed=2)
    xbuf = torch.empty(n + 4, dtype=torch.float32, device=dev)
    xbuf[:n].copy_(x_host)
    xbuf[n:].zero_()
    x = xbuf[:n]
    y = torch.empty(n, dtype=torch.float32, device=dev)
    S, T, TPB = args.stages, args.tile, args.tiles_per_block
    alg_bytes = 8 * n
    path = tp.pipelined_map(x, y, "scale2", T, S, TPB)
    plan = tp.plan_map(x.data_ptr(), y.data_ptr(), n, "scale2", T, S, TPB)
    torch.cuda.synchronize()
    parity = sampled_parity(x_host, y, "scale2")
    log(f"headline parity (sampled windows vs oracle): {parity}")
    step = lambda: tp.pipelined_map(x, y, "scale2", T, S, TPB)
    gpu_warmup(step)
    region = time_region(step, args.warmup, args.steps)          # the whole job, back to back
    per, _ = time_launches(step, 2, args.steps)                   # per-launch kernel durations
    ms_step = region / args.steps
    value = alg_bytes / (ms_step * 1e-3) / 1e9
    avg_launch = sum(per) / len(per)
    achieved = alg_bytes / (avg_launch * 1e-3) / 1e9
    log(f"headline: {value:.1f} GB/s ({100 * value / HBM_PEAK_GBS:.1f}% of peak), "
        f"avg launch {avg_launch * 1e3:.1f} us")

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"pipelined scale-by-2 map over 2^28 fp32 (1 GiB in, 1 GiB out), "
                               f"uniform [-1,1) seed 2, tile {T} fp32, {S} stages, "
                               f"{plan.tiles_per_block} tiles per workgroup, 16-byte path",
                   "n": n, "tile_elems": T, "stages": S, "tiles_per_block": plan.tiles_per_block,
                   "grid": plan.grid, "path": tp.Path(path).name.lower(),
                   "resident_workgroups_per_cu": plan.resident_cap or None,
                   "lds_bytes_per_workgroup": plan.lds_bytes},
        "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "parity": "bit-exact on sampled windows" if parity else "MISMATCH",
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": stored_traffic(step_traffic_key(n, T, S, plan.tiles_per_block)),
                     "kernel": "map_kernel<scale2>", "algorithmic_bytes_per_launch": alg_bytes,
                     "avg_launch_us": round(avg_launch * 1e3, 2)},
    }

    # copy ceiling for context: the runtime's device-to-device copy of 1 GiB
    per_c, _ = time_launches(lambda: y.copy_(x), 3, 10)
    result["copy_ceiling_GBs"] = round(alg_bytes / (median(per_c) * 1e-3) / 1e9, 1)

    if not args.quick:
        result["rows"] = extra_rows(args, tp, workloads, torch, np, dev, x_host, xbuf, y)

    if not args.no_cpu_baseline:
        log("cpu baseline: oracle scale2 on the host cores")
        result["cpu_baseline"] = cpu_baseline(x_host, "scale2", 8, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


MAP2D_ROWS, MAP2D_COLS, MAP2D_SRC_STRIDE = 16384, 16384, 16448
MAP2D_BOXES = [(1, 256), (4, 256), (1, 1024), (2, 512), (8, 128), (16, 64), (4, 1024)]


def map_2d_row(tp, workloads, torch, np, dev, scratch):
    """scale2 over a 16384 x 16384 fp32 window (1 GiB) of a source whose rows
    are 16448 floats apart, into a dense destination, for several box shapes
    at 2 stages and runs of 2; sampled rows checked against the oracle."""
    import oracle
    R, C, SS = MAP2D_ROWS, MAP2D_COLS, MAP2D_SRC_STRIDE
    src_h = workloads.uniform_pm1(R * SS, seed=6)
    src = src_h.to(dev).view(R, SS)[:, :C]
    dst = torch.empty(R, C, dtype=torch.float32, device=dev)
    out = {"workload": f"scale2 over a {R} x {C} fp32 window (row stride {SS}) into a dense "
                       f"{R} x {C} destination; 2 stages, runs of 2 boxes", "boxes": {}}
    gpu_warmup(lambda: tp.map_2d(src, dst, "scale2", 4, 256, 2, 0))
    for br, bc in MAP2D_BOXES:
        f = lambda: tp.map_2d(src, dst, "scale2", br, bc, 2, 0)
        f()
        per, _ = time_launches(f, 2, 10)
        gbs = 8 * R * C / (median(per) * 1e-3) / 1e9
        out["boxes"][f"{br}x{bc}"] = {"GBs": round(gbs, 1), "pct_peak": round(100 * gbs / HBM_PEAK_GBS, 1)}
    # parity of the last launch on sampled rows
    rng = np.random.default_rng(0)
    sh = src_h.numpy().reshape(R, SS)
    ok = True
    for r in rng.integers(0, R, size=12):
        exp = oracle.pipelined_map(sh[r, :C], "scale2", threads=1)
        ok &= bool(np.array_equal(dst[r].cpu().numpy().view(np.uint32), exp.view(np.uint32)))
    out["parity_sampled_rows"] = ok
    del src, dst
    log(f"map_2d: {out['boxes']}")
    return out


def extra_rows(args, tp, workloads, torch, np, dev, x_host, xbuf, y):
    rows = {}
    n = x_host.numel()

    # stage/tile sweep, aligned and with a 4-byte source offset (16-byte loads at
    # that offset, and the pages' 4-byte fallback)
    sweep = []
    shifted = torch.cat([x_host[1:], torch.zeros(1)])[:n]
    parity = True
    gpu_warmup(lambda: tp.pipelined_map(xbuf[:n], y, "scale2", 256, 2, 0))
    for off, align, T, S in sweep_points():
        xin = xbuf[off:off + n]
        f = lambda: tp.pipelined_map(xin, y, "scale2", T, S, 0, align=align)
        p = f()
        per, _ = time_launches(f, 2, 8)
        gbs = 8 * n / (median(per) * 1e-3) / 1e9
        sweep.append({"src_offset_bytes": 4 * off, "align": align, "tile": T, "stages": S,
                      "path": tp.Path(p).name.lower(), "GBs": round(gbs, 1),
                      "pct_peak": round(100 * gbs / HBM_PEAK_GBS, 1)})
        if off and S == 4 and T == 1024:
            parity &= bool(sampled_parity(shifted, y, "scale2"))
    log("sweep done")
    rows["sweep_parity_offset4"] = parity
    rows["scale2_sweep"] = sweep

    # the output 4 bytes past a 128-byte boundary, the case the 4-byte fallback
    # serves worst: realigned (the first 31 floats element-wise, then 16-byte
    # stores that fill whole lines) against the pages' fallback
    ybuf = torch.empty(n + 4, dtype=torch.float32, device=dev)
    yout = ybuf[1:n + 1]
    mis = {}
    for align in ("realign", "words"):
        f = lambda: tp.pipelined_map(xbuf[:n], yout, "scale2", 256, 2, 0, align=align)
        p = f()
        per, _ = time_launches(f, 2, 10)
        gbs = 8 * n / (median(per) * 1e-3) / 1e9
        mis[align] = {"path": tp.Path(p).name.lower(), "GBs": round(gbs, 1),
                      "pct_peak": round(100 * gbs / HBM_PEAK_GBS, 1),
                      "parity": bool(sampled_parity(x_host, yout, "scale2"))}
    rows["scale2_output_offset4"] = dict(mis, workload="scale2 over 2^28 floats, tile 256, 2 stages, "
                                                       "output 4 bytes past a 128-byte boundary")
    log(f"output offset 4 B: {mis}")
    del ybuf, yout

    # small double-buffered map: 2^24, tile 256, 2 stages, 64 tiles per workgroup
    ns = 1 << 24
    xs_host = workloads.uniform_pm1(ns, seed=1)
    xs = xs_host.to(dev)
    ys = torch.empty_like(xs)
    small = lambda: tp.pipelined_map(xs, ys, "scale2", 256, 2, 64)
    gpu_warmup(small)
    per, _ = time_launches(small, 5, 50)
    warm = 8 * ns / (median(per) * 1e-3) / 1e9
    # the same launch with the caches flushed first: 1 GiB written to another
    # buffer between repetitions evicts the 128 MiB footprint from the 256 MB
    # Infinity Cache and the L2s; only the map launch is between the events
    s = torch.cuda.current_stream()
    cold = []
    for _ in range(20):
        y.fill_(0.0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        small()
        e1.record(s)
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    flushed = 8 * ns / (median(cold) * 1e-3) / 1e9
    rows["scale2_small"] = {"n": ns, "tile": 256, "stages": 2, "tiles_per_block": 64,
                            "GBs_cache_warm": round(warm, 1), "GBs_flushed": round(flushed, 1),
                            "us_cache_warm": round(median(per) * 1e3, 2),
                            "us_flushed": round(median(cold) * 1e3, 2),
                            "note": "1 024 one-wave workgroups (64 tiles each): latency-bound by the "
                                    "configuration; the 128 MiB footprint fits the Infinity Cache"}
    log(f"scale2 small: warm {warm:.0f} GB/s, flushed {flushed:.0f} GB/s")
    del xs, ys

    # compute-heavy map: 2^27, horner32, stages 1/2/4
    nh = 1 << 27
    xh_host = workloads.uniform_pm1(nh, seed=4)
    xh = xh_host.to(dev)
    yh = torch.empty_like(xh)
    hr = {}
    # (tile, tiles per workgroup, bound on resident workgroups per CU):
    # tile 1024 (the workload's tile) at the library's run length and at 16
    # tiles per workgroup, tile 256 (one-wave workgroups) at the library's run,
    # and tile 1024 with 8 tiles per workgroup at 2 workgroups (8 waves) per CU,
    # the occupancy of a kernel whose registers or LDS leave few waves resident
    # ... each with every wave loading its own part (uniform), and the first
    # and last also with one wave doing all loads for the others (role split)
    groups = [(1024, 0, 0, "uniform"), (1024, 16, 0, "uniform"), (256, 0, 0, "uniform"),
              (1024, 8, 2, "uniform"), (1024, 0, 0, "role_split"), (1024, 8, 2, "role_split")]
    configs = [(tile, tpb, cap, sched, S) for tile, tpb, cap, sched in groups for S in (1, 2, 4)]
    run = lambda tile, tpb, cap, sched, S: tp.pipelined_map(xh, yh, "horner32", tile, S, tpb,
                                                            resident_cap=cap, schedule=sched)
    for c in configs:
        run(*c)
    gpu_warmup(lambda: run(1024, 0, 0, "uniform", 2))
    # the configurations take turns over several rounds, so that a drift of the
    # clocks during the run does not favour whichever ran first
    times = {c: [] for c in configs}
    for _ in range(6):
        for c in configs:
            per, _ = time_launches(lambda: run(*c), 1, 4)
            times[c] += per
    name = lambda tile, tpb, cap, sched: (("" if tile == 1024 else f"tile{tile}_")
                                          + f"T{tpb or 'default'}"
                                          + (f"_{cap}wg_per_cu" if cap else "")
                                          + ("_role_split" if sched == "role_split" else ""))
    for tile, tpb, cap, sched, S in configs:
        t = median(times[(tile, tpb, cap, sched, S)]) * 1e-3
        hr[f"{name(tile, tpb, cap, sched)}_S{S}"] = {"GBs": round(8 * nh / t / 1e9, 1),
                                                     "TFLOPs": round(64 * nh / t / 1e12, 2),
                                                     "us": round(t * 1e6, 1)}
    for tile, tpb, cap, sched in groups:
        key = name(tile, tpb, cap, sched)
        hr[f"{key}_speedup_S2_over_S1"] = round(hr[f"{key}_S1"]["us"] / hr[f"{key}_S2"]["us"], 3)
        hr[f"{key}_speedup_S4_over_S1"] = round(hr[f"{key}_S1"]["us"] / hr[f"{key}_S4"]["us"], 3)
    hr["parity"] = bool(sampled_parity(xh_host, yh, "horner32"))
    hr["fp32_valu_peak_TFLOPs"] = FP32_VALU_PEAK_TFLOPS
    rows["horner32"] = hr
    log(f"horner32: {hr}")
    del xh, yh

    # memory-bound map (scale2 over the step's input) at 1/2/4 stages: the
    # library's launch, and tile 1024 in runs of 8 at 2 workgroups (8 waves)
    # per CU, where other waves no longer hide a wave's loads; interleaved rounds
    xm = xbuf[:n]
    sgroups = [(256, 0, 0), (1024, 8, 2)]
    sconf = [(tile, tpb, cap, S) for tile, tpb, cap in sgroups for S in (1, 2, 4)]
    srun = lambda tile, tpb, cap, S: tp.pipelined_map(xm, y, "scale2", tile, S, tpb, resident_cap=cap)
    gpu_warmup(lambda: srun(256, 0, 0, 2))
    st = {c: [] for c in sconf}
    for _ in range(4):
        for c in sconf:
            per, _ = time_launches(lambda: srun(*c), 1, 4)
            st[c] += per
    sr = {}
    for tile, tpb, cap in sgroups:
        key = f"tile{tile}_T{tpb or 'default'}" + (f"_{cap}wg_per_cu" if cap else "_library_bound")
        for S in (1, 2, 4):
            t = median(st[(tile, tpb, cap, S)]) * 1e-3
            sr[f"{key}_S{S}"] = {"GBs": round(8 * n / t / 1e9, 1), "us": round(t * 1e6, 1)}
        sr[f"{key}_speedup_S2_over_S1"] = round(sr[f"{key}_S1"]["us"] / sr[f"{key}_S2"]["us"], 3)
        sr[f"{key}_speedup_S4_over_S1"] = round(sr[f"{key}_S1"]["us"] / sr[f"{key}_S4"]["us"], 3)
    sr["parity"] = bool(sampled_parity(x_host, y, "scale2"))
    rows["scale2_stages"] = sr
    log(f"scale2 stages: {sr}")

    # vendor kernels on the same 1 GiB buffers, for context: a read-only
    # reduction (torch.sum reads 1 GiB) and a write-only fill (1 GiB written)
    xr = xbuf[:n]
    gpu_warmup(lambda: xr.sum())
    per_r, _ = time_launches(lambda: xr.sum(), 2, 10)
    per_w, _ = time_launches(lambda: y.fill_(1.0), 2, 10)
    rows["vendor_context"] = {
        "torch_sum_read_only_GBs": round(4 * n / (median(per_r) * 1e-3) / 1e9, 1),
        "torch_fill_write_only_GBs": round(4 * n / (median(per_w) * 1e-3) / 1e9, 1),
        "note": "torch.sum over the step's 1 GiB input and fill_ of its 1 GiB output, "
                "bytes moved per second; the runtime's 1 GiB copy is copy_ceiling_GBs"}
    log(f"vendor context: {rows['vendor_context']}")

    rows["map_2d"] = map_2d_row(tp, workloads, torch, np, dev, y)

    # predicated chunk copy: 2^26 chunks
    rows["chunk_copy"] = chunk_copy_row(tp, workloads, torch, np, dev, args.cpu_seconds)

    rows["workgroup_copy"] = workgroup_copy_row(tp, torch, np, dev)

    # row exchange 64x4 (launch-bound)
    a = workloads.arange_rows(64).to(dev)
    b = torch.empty_like(a)
    per, region = time_launches(lambda: tp.row_shift(a, b), 10, 1000)
    # the same 1000 launches captured once in a HIP graph and replayed: the
    # time per kernel without the host's per-call work
    g = torch.cuda.CUDAGraph()
    tp.row_shift(a, b)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for _ in range(1000):
            tp.row_shift(a, b)
    g.replay()
    torch.cuda.synchronize()
    graph_ms = time_region(g.replay, 2, 5) / 5
    rows["row_shift"] = {"rows": 64, "median_launch_us": round(median(per) * 1e3, 2),
                         "region_us_per_call": round(region, 4),
                         "graph_replay_us_per_kernel": round(graph_ms, 4)}
    ok = np.array_equal(b.cpu().numpy().view(np.uint32),
                        __import__("oracle").row_shift(a.cpu().numpy()).view(np.uint32))
    rows["row_shift"]["parity"] = bool(ok)
    return rows


if __name__ == "__main__":
    main()
