"""Host-side checks of bench.py that need no GPU: the one-GPU contract, the
algorithmic byte count of the chunk copy, and the ordering property the
hardware-counter summaries rely on."""
import importlib.util
import os
import subprocess
import sys

import software_pipelining_amd as tp
from software_pipelining_amd import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_chunk_copy_algorithmic_bytes_brute_force():
    # per chunk: 3 metadata bytes, the kept source prefix of a written chunk,
    # and 16 bytes written when pred is set
    bench = _bench()
    inp = workloads.chunk_copy_inputs(5000, seed=9, sizes=tuple(range(0, 20)))
    want = 0
    for p, s, g in zip(inp.pred.tolist(), inp.src_size.tolist(), inp.ignore_src.tolist()):
        want += 3
        if p:
            want += 16 + (0 if g else min(s, 16))
    assert bench.chunk_copy_algorithmic_bytes(inp.pred, inp.src_size, inp.ignore_src) == want


def test_chunk_copy_bytes_per_chunk_near_expectation():
    # E[bytes] = 3 + 0.9 * 0.99 * 8 + 0.9 * 16 = 24.528 for the workload's draws
    bench = _bench()
    inp = workloads.chunk_copy_inputs(1 << 20, seed=3)
    per_chunk = bench.chunk_copy_algorithmic_bytes(inp.pred, inp.src_size, inp.ignore_src) / (1 << 20)
    assert abs(per_chunk - 24.528) < 0.05


def test_sweep_points_are_told_apart_by_order():
    # consecutive points never launch the same kernel on the same grid, so the
    # per-point counter summaries can split dispatches by order
    bench = _bench()
    pts = bench.sweep_points()
    assert len(pts) == len(set(pts)) == 36
    A, B = 0x7f0000000000, 0x7f4000000000
    keys = []
    for off, align, tile, stages in pts:
        p = tp.plan_map(A + 4 * off, B, 1 << 28, "scale2", tile, stages, 0, align=align)
        keys.append((stages, p.lane_chunks, p.path, p.grid, p.threads))
    assert all(a != b for a, b in zip(keys, keys[1:]))


def test_stored_traffic_is_tied_to_the_sources():
    bench = _bench()
    h = bench.kernel_source_hash()
    assert len(h) == 16 and int(h, 16) >= 0
    entry = bench.stored_traffic("map_scale2_n268435456_t256_s2_T4")
    # either the stored counters describe the current sources, or nothing is reported
    assert entry is None or 2 * (1 << 30) <= entry < 2 * (1 << 30) * 1.01


def _counter_csv(path, counter, map_kib, copy_kib):
    import csv
    os.makedirs(os.path.dirname(path), exist_ok=True)
    cols = ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(cols)
        for i in range(3):
            w.writerow([i, 1 << 25, "void tp::dev::map_kernel<0, 2, 1, true, true>(tp::MapParams)",
                        counter, map_kib])
        w.writerow([7, 1 << 25, "void tp::dev::map_kernel<1, 2, 1, true, true>(tp::MapParams)",
                    counter, 1.0])
        w.writerow([8, 1 << 25, "__amd_rocclr_copyBuffer", counter, copy_kib])   # the 1 GiB copy
        w.writerow([9, 4096, "__amd_rocclr_copyBuffer", counter, 5.0])          # a staging copy


def test_record_traffic_scales_by_the_copy(tmp_path):
    # FETCH_SIZE reads half of a known 1 GiB copy, WRITE_SIZE all of it: the
    # map's readings are scaled by 2 and 1, and the entry carries the hash of
    # the sources it describes
    bench = _bench()
    _counter_csv(str(tmp_path / "f" / "h" / "1" / "x_counter_collection.csv"), "FETCH_SIZE",
                 524300.0, 524288.0)
    _counter_csv(str(tmp_path / "w" / "h" / "1" / "x_counter_collection.csv"), "WRITE_SIZE",
                 1048576.0, 1048576.0)
    out = str(tmp_path / "traffic.json")
    bench.record_traffic(str(tmp_path / "f"), str(tmp_path / "w"), out)
    plan = tp.plan_map(1 << 40, 1 << 41, 1 << 28, "scale2", 256, 2, 0)
    key = bench.step_traffic_key(1 << 28, 256, 2, plan.tiles_per_block)
    got = bench.stored_traffic(key, out)
    assert got == 2 * 524300 * 1024 + 1048576 * 1024
    import json
    with open(out) as f:
        e = json.load(f)[key]
    assert e["scale"] == {"FETCH_SIZE": 2.0, "WRITE_SIZE": 1.0}
    assert e["kernel_source_hash"] == bench.kernel_source_hash()


def test_record_chunk_traffic_groups_dispatches_by_order(tmp_path):
    # the chunk-copy dispatches of `--mode chunk` fall in one group per point
    # of CHUNK_COUNTER_POINTS (one untimed launch, then the timed ones): each
    # point's bytes are the median of its timed launches, calibrated on the
    # runtime's 1 GiB copy, and the entry is tied to the chunk copy's sources
    import csv
    import json
    bench = _bench()
    pts = bench.CHUNK_COUNTER_POINTS
    for counter, sub, copy_kib in (("FETCH_SIZE", "f", 524288.0), ("WRITE_SIZE", "w", 1048576.0)):
        path = tmp_path / sub / "x_counter_collection.csv"
        os.makedirs(path.parent, exist_ok=True)
        with open(path, "w", newline="") as f:
            w = csv.writer(f)
            w.writerow(["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value"])
            did = 0
            for i, _ in enumerate(pts):
                for j in range(4):          # untimed launch (a stray value), then 3 timed
                    val = 9e9 if j == 0 else 1000.0 * (i + 1) + j
                    w.writerow([did, 1 << 18, "void tp::dev::chunk_copy_kernel<1, 16, true, true>",
                                counter, val])
                    did += 1
            w.writerow([did, 1 << 25, "__amd_rocclr_copyBuffer", counter, copy_kib])
    out = str(tmp_path / "traffic.json")
    bench.record_chunk_traffic(str(tmp_path / "f"), str(tmp_path / "w"), out)
    with open(out) as f:
        table = json.load(f)
    for i, (operands, stages, tpb) in enumerate(pts):
        plan = tp.plan_chunk_copy(1 << 40, 1 << 41, 1 << 26, stages=stages, tiles_per_block=tpb)
        e = table[bench.chunk_traffic_key(operands, plan.stages, plan.tiles_per_block)]
        mid = 1000.0 * (i + 1) + 2          # median of the three timed launches
        assert e["fetch_bytes"] == round(mid * 2 * 1024) and e["write_bytes"] == round(mid * 1024)
        assert e["kernel_source_hash"] == bench.kernel_source_hash(bench.CHUNK_KERNEL_SOURCES)
    assert len({bench.chunk_traffic_key(o, *(lambda p: (p.stages, p.tiles_per_block))(
        tp.plan_chunk_copy(1 << 40, 1 << 41, 1 << 26, stages=s, tiles_per_block=t)))
        for o, s, t in pts}) == len(pts)
