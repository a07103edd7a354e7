"""Host-side checks of libtilepipe that need no GPU: the shared library loads,
exports every symbol include/tilepipe.h declares, and its planner enforces the
documented argument rules (null pointers, sizes, alignment, overlap, LDS
budget) and launch geometry. Only host-only calls are made here."""
import ctypes
import os
import re

import pytest

import software_pipelining_amd as tp
from software_pipelining_amd import tilepipe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tilepipe.h")

BIG = 1 << 62                 # "no LDS limit" for pure argument checks
A = 0x7f0000000000            # fake, well-aligned device addresses
B = 0x7f4000000000


def _declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"TP_API\s+[\w\s\*]*?\b(tp_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = tilepipe._load()
    names = _declared_symbols()
    assert len(names) >= 10
    for name in names:
        assert hasattr(lib, name), name
    assert lib.tp_version() == 1


def test_status_strings():
    lib = tilepipe._load()
    for code, name in enumerate(tilepipe._STATUS):
        assert lib.tp_status_string(code).decode() == name
    assert lib.tp_status_string(99).decode() == "TP_ERR_UNKNOWN"


def _status(fn, *args, **kwargs):
    try:
        fn(*args, **kwargs)
        return 0
    except tp.TilepipeError as e:
        return e.status


# ------------------------------------------------------------------ map
def test_map_plan_geometry_runs():
    for tile, threads, lanes in [(256, 64, 1), (512, 128, 1), (1024, 256, 1), (2048, 256, 2),
                                 (4096, 256, 4), (8192, 256, 8)]:
        p = tp.plan_map(A, B, 1 << 20, "scale2", tile, 2, 64)
        assert (p.threads, p.lane_chunks, p.tiles_per_block) == (threads, lanes, 64)
        assert p.num_tiles == (1 << 20) // tile
        assert p.grid == -(-p.num_tiles // 64)
        assert p.ring_bytes == 2 * tile * 4 + 256
        assert p.lds_bytes >= p.ring_bytes
        assert p.path == tp.Path.X4


def test_map_plan_default_run_length():
    # runs of 4 tiles of at most 512 floats (4-8 KiB), of 2 larger tiles
    p = tp.plan_map(A, B, 1 << 28, "scale2", 256, 2, 0)
    assert p.tiles_per_block == 4 and p.grid == (1 << 20) // 4
    for tile, run in ((512, 4), (1024, 2), (2048, 2), (8192, 2)):
        assert tp.plan_map(A, B, 1 << 28, "horner32", tile, 2, 0).tiles_per_block == run, tile
    # the same whatever the alignment of the input
    assert tp.plan_map(A + 4, B, 1 << 28, "scale2", 256, 2, 0).tiles_per_block == 4
    p = tp.plan_map(A, B, 5000, "scale2", 1024, 2, 0)
    assert (p.num_tiles, p.grid) == (5, 3)
    # the 2-D map keeps runs of 2 boxes
    assert tp.plan_map_2d(A, 1024, B, 1024, 64, 1024, "scale2", 1, 256).tiles_per_block == 2
    # the chunk copy's default run is max(S-1, m) tiles, m = 1, 2, 8 for 16-,
    # 8- and 4-byte chunks: with 16-byte chunks the prologue holds the whole run
    for width, stages, run in ((16, 1, 1), (16, 2, 1), (16, 3, 2), (16, 4, 3), (16, 8, 7),
                               (8, 1, 2), (8, 2, 2), (8, 4, 3), (4, 2, 8), (4, 8, 8)):
        p = tp.plan_chunk_copy(A, B, 1 << 26, stages=stages, chunk_bytes=width)
        assert p.tiles_per_block == run, (width, stages)


def test_map_plan_tail_and_small_sizes():
    assert tp.plan_map(A, B, 0).grid == 0
    p = tp.plan_map(A, B, 3, tile_elems=1024, tiles_per_block=64)
    assert (p.num_tiles, p.grid) == (0, 1)          # tail-only launch
    p = tp.plan_map(A, B, 1027, tile_elems=1024, tiles_per_block=1)
    assert (p.num_tiles, p.grid) == (1, 1)          # one tile, then a 3-float tail
    p = tp.plan_map(A, B, 1029, tile_elems=1024, tiles_per_block=1)
    assert (p.num_tiles, p.grid) == (2, 2)          # a partial second tile, 1-float tail
    p = tp.plan_map(A, B, (1 << 28), tile_elems=256, stages=2, tiles_per_block=64)
    assert p.grid == 16384


def test_map_plan_paths_follow_alignment():
    # the pages' rule: 4-byte words on a side that is not 16-byte aligned
    w = dict(align="words")
    assert tp.plan_map(A + 4, B, 100, **w).path == tp.Path.SCALAR_LOAD
    assert tp.plan_map(A, B + 8, 100, **w).path == tp.Path.SCALAR_STORE
    assert tp.plan_map(A + 12, B + 4, 100, **w).path == tp.Path.SCALAR
    assert tp.plan_map(A + 16, B + 32, 100, **w).path == tp.Path.X4
    assert tp.plan_map(A + 12, B + 4, 100, **w).head == 0
    assert tp.plan_map(A + 12, B + 4, 100, **w).align == tp.Align.WORDS


def test_map_plan_realign():
    # the default: 16-byte accesses at any 4-byte alignment, the tiled body
    # starting at out's first 128-byte boundary (A and B are 128-byte aligned)
    assert A % 128 == 0 and B % 128 == 0
    n = 5000
    for in_off in (0, 4, 8, 12, 64, 68):
        for out_off in (0, 4, 8, 12, 16, 64, 124):
            # out's boundary, or in's when out - in is 64 mod 128 (half-line stores)
            anchor = in_off if (out_off - in_off) % 128 == 64 else out_off
            head = (128 - anchor) % 128 // 4
            p = tp.plan_map(A + in_off, B + out_off, n, tile_elems=1024, tiles_per_block=1)
            assert (p.path, p.head, p.align) == (tp.Path.X4, head, tp.Align.REALIGN)
            n_main = (n - head) // 4 * 4
            assert (p.num_tiles, p.grid) == (-(-n_main // 1024), -(-n_main // 1024))
    # fewer floats than the distance to the boundary: all of them are the head
    for n in (1, 2, 3, 30, 31):
        p = tp.plan_map(A, B + 4, n)
        assert (p.head, p.num_tiles, p.grid) == (n, 0, 1)
    p = tp.plan_map(A, B + 4, 32)
    assert (p.head, p.num_tiles, p.grid) == (31, 0, 1)          # a 1-float tail
    p = tp.plan_map(A, B + 4, 31 + 1024, tile_elems=1024, tiles_per_block=1)
    assert (p.head, p.num_tiles, p.grid) == (31, 1, 1)
    p = tp.plan_map(A, B + 120, 2 + 1023, tile_elems=1024, tiles_per_block=1)
    assert (p.head, p.num_tiles, p.grid) == (2, 1, 1)           # 1020-float body, 3-float tail
    assert tp.plan_map(A, B, 0).head == 0 and tp.plan_map(0, 0, 0, "scale2").grid == 0
    # the realigned launch waits like the 16-byte path; in place keeps one head
    assert tp.plan_map(A + 4, B + 4, 100, stages=2).wait_steady == 1 + 1
    assert tp.plan_map(A + 8, A + 8, 100).head == 30
    assert tp.plan_map(A, B + 64, 100).head == 0                  # stores at half lines
    assert tp.plan_map(A + 4, B + 68, 100).head == 31             # in's boundary
    assert tp.plan_map(B + 68, A + 4, 100).head == 15
    assert tp.plan_map(A + 64, B, 100).head == 16                 # out - in = -64 = 64 mod 128
    for bad in (2, -1):
        assert _status(tp.plan_map, A, B, 10, align=bad) == 1


def test_map_plan_wait_counts():
    # steady-state vmcnt between a tile's last load and its wait, per lane:
    # matching widths refill before waiting, (S-1) loads + (S-1) stores;
    # mixed widths wait before the barrier and refill, (S-2) loads + (S-1) stores;
    # 0 for S = 1; clamped to 63
    assert tp.plan_map(A, B, 100, stages=1).wait_steady == 0
    assert tp.plan_map(A, B, 100, stages=2).wait_steady == 1 + 1
    assert tp.plan_map(A, B, 100, stages=4, tile_elems=4096).wait_steady == 3 * 4 + 3 * 4
    assert tp.plan_map(A + 4, B + 4, 100, stages=2, tile_elems=1024,
                       align="words").wait_steady == 4 + 4
    w = dict(align="words")
    assert tp.plan_map(A + 4, B, 100, stages=1, tile_elems=1024, **w).wait_steady == 0
    assert tp.plan_map(A + 4, B, 100, stages=3, tile_elems=1024, **w).wait_steady == 4 + 2
    assert tp.plan_map(A, B + 4, 100, stages=2, tile_elems=2048, **w).wait_steady == 0 + 8
    assert tp.plan_map(A + 4, B + 4, 100, stages=8, tile_elems=8192, **w).wait_steady == 63


@pytest.mark.parametrize("args,status", [
    ((A, B, -1), 1),
    ((0, B, 10), 1),
    ((A, 0, 10), 1),
    ((A + 2, B, 10), 2),
    ((A, B + 1, 10), 2),
    ((A, A + 4, 10), 4),          # partial overlap
    ((A + 36, A, 10), 4),
])
def test_map_plan_argument_errors(args, status):
    assert _status(tp.plan_map, *args) == status


def test_map_plan_option_errors():
    assert _status(tp.plan_map, A, B, 10, "nope") == 1
    for tile in (0, 64, 128, 300, 16384):
        assert _status(tp.plan_map, A, B, 10, "scale2", tile) == 1
    for s in (0, 9, -1):
        assert _status(tp.plan_map, A, B, 10, "scale2", 1024, s) == 1
    assert _status(tp.plan_map, A, B, 10, "scale2", 1024, 2, -1) == 1
    assert _status(tp.plan_map, A, B, 10, "scale2", 1024, 2, 65537) == 1
    assert _status(tp.plan_map, A, B, 10, "scale2", 8192, 2, 65536) == 1   # run > 1 GiB
    assert _status(tp.plan_map, A, B, 10, "scale2", 1024, 2, -3) == 1
    assert _status(tp.plan_map, A, B, 1 << 41) == 1
    # 2^40 floats in 256-float tiles, runs of one: 2^32 workgroups, more than a launch names
    far_a, far_b = 1 << 44, 1 << 45                                        # 4 TiB buffers
    assert _status(tp.plan_map, far_a, far_b, 1 << 40, "scale2", 256, 1, 1) == 1
    assert _status(tp.plan_map, far_a, far_b, 1 << 40, "scale2", 256, 1, 2) == 1   # 2^31 WGs
    assert tp.plan_map(far_a, far_b, 1 << 40, "scale2", 256, 1, 4).grid == 1 << 30
    # exact aliasing is allowed; n == 0 accepts null pointers
    assert tp.plan_map(A, A, 10).grid == 1
    assert tp.plan_map(0, 0, 0).grid == 0


def test_map_plan_lds_budget():
    assert _status(tp.plan_map, A, B, 10, "scale2", 4096, 4, 0, 64 * 1024) == 3
    assert tp.plan_map(A, B, 10, "scale2", 4096, 4, 0, 160 * 1024).ring_bytes == 4 * 16384 + 256
    assert tp.plan_map(A, B, 10, "horner32", 4096, 4, 0, 160 * 1024).lds_bytes == 4 * 16384 + 256
    assert _status(tp.plan_map, A, B, 10, "scale2", 8192, 8, 0, 160 * 1024) == 3


KIB = 1024


def _reserve(cap, ring, budget=160 * KIB):
    return max(ring, min(budget, (160 * KIB // cap) // KIB * KIB))


def test_map_residency_policy_values():
    # worked by hand from the rule: cap = round(27 KiB (1 + 1/T) / ((a + 1) tile bytes)),
    # a = mean over the run of min(S, tiles left), at least 4 workgroups and 8 waves
    cases = [  # tile, S, T, cap
        (256, 2, 4, 12),     # the step: a = 1.75: 34560 / (2.75 * 1024) = 12.3
        (256, 2, 2, 16),     # a = 1.5: 41472 / (2.5 * 1024) = 16.2
        (256, 1, 2, 20),     # a = 1: 41472 / 2048 = 20.3
        (256, 4, 8, 8),      # a = 26/8: 31104 / (4.25 * 1024) = 7.1 -> 7, raised to 8 waves
        (1024, 2, 2, 4),     # 41472 / (2.5 * 4096) = 4.05
        (1024, 4, 8, 4),     # 31104 / (4.25 * 4096) = 1.8, raised to 4 workgroups
        (512, 4, 4, 5),      # a = 2.5: 34560 / (3.5 * 2048) = 4.8
        (2048, 2, 2, 0),     # two 16-byte loads per lane per tile: not bounded
        (4096, 4, 2, 0),
    ]
    for tile, S, T, cap in cases:
        p = tp.plan_map(A, B, 1 << 26, "scale2", tile, S, T)
        assert p.resident_cap == cap, (tile, S, T, p.resident_cap)
        assert p.lds_bytes == (_reserve(cap, p.ring_bytes) if cap else p.ring_bytes)
        assert tp.plan_map(A, B, 1 << 26, "copy", tile, S, T).resident_cap == cap


def test_map_residency_policy_rules():
    for tile in (256, 1024, 4096):
        for S in (1, 2, 4):
            for T in (1, 2, 16):
                h = tp.plan_map(A, B, 1 << 26, "horner32", tile, S, T)
                assert (h.resident_cap, h.lds_bytes) == (0, h.ring_bytes)   # compute-heavy: none
                p = tp.plan_map(A, B, 1 << 26, "scale2", tile, S, T)
                if T == 1:
                    assert p.resident_cap == 0                       # no pipeline to bound
                waves = p.threads // 64
                if tile > 1024:
                    assert p.resident_cap == 0
                if p.resident_cap:
                    assert p.resident_cap * waves >= 8 and p.resident_cap >= 4
                    assert p.resident_cap < 32 // waves              # below the hardware limit
                    assert p.lds_bytes == _reserve(p.resident_cap, p.ring_bytes)
                    assert 160 * KIB // p.lds_bytes >= p.resident_cap
                else:
                    assert p.lds_bytes == p.ring_bytes
    # deeper pipelines and bigger tiles never get more resident workgroups
    for T in (2, 4, 16):
        caps = [tp.plan_map(A, B, 1 << 26, "scale2", 256, S, T).resident_cap or 32 for S in (1, 2, 3, 4)]
        assert caps == sorted(caps, reverse=True), (T, caps)
        caps = [tp.plan_map(A, B, 1 << 26, "scale2", t, 2, T).resident_cap or 32 // max(1, t // 256)
                for t in (256, 512, 1024, 2048)]
        assert caps == sorted(caps, reverse=True), (T, caps)


def test_map_explicit_residency():
    ring = 2 * 1024 * 4 + 256
    p = tp.plan_map(A, B, 1 << 20, "scale2", 1024, 2, 2, resident_cap=-1)
    assert (p.resident_cap, p.lds_bytes) == (0, ring)
    for cap in (1, 2, 3, 5, 7):
        p = tp.plan_map(A, B, 1 << 20, "horner32", 1024, 2, 2, resident_cap=cap)
        assert (p.resident_cap, p.lds_bytes) == (cap, _reserve(cap, ring))
    # at or above the hardware's own limit (8 workgroups of 4 waves): nothing to reserve
    p = tp.plan_map(A, B, 1 << 20, "scale2", 1024, 2, 2, resident_cap=8)
    assert (p.resident_cap, p.lds_bytes) == (0, ring)
    # the reservation never exceeds the budget, and the ring still decides the error
    p = tp.plan_map(A, B, 1 << 20, "scale2", 1024, 2, 2, 32 * KIB, resident_cap=1)
    assert p.lds_bytes == 32 * KIB
    p = tp.plan_map(A, B, 1 << 20, "scale2", 4096, 8, 2, resident_cap=2)     # ring > 80 KiB
    assert p.lds_bytes == 8 * 16384 + 256
    assert _status(tp.plan_map, A, B, 10, "scale2", 1024, 2, 2, tilepipe._NO_BUDGET, -2) == 1


def test_map_role_split_plan():
    # one more wave that only loads; its wait counts only its own loads of the
    # S-2 tiles issued after the waited one (it issues no stores)
    for tile, threads, per_tile in [(256, 128, 1), (512, 192, 2), (1024, 320, 4), (2048, 320, 8),
                                    (4096, 320, 16), (8192, 320, 32)]:
        for S in (1, 2, 3, 4):
            p = tp.plan_map(A, B, 1 << 20, "horner32", tile, S, 2, schedule="role_split")
            assert p.schedule == tp.Schedule.ROLE_SPLIT and p.threads == threads
            assert p.wait_steady == min(63, (S - 2) * per_tile) if S > 1 else p.wait_steady == 0
            q = tp.plan_map(A + 4, B, 1 << 20, "horner32", tile, S, 2, schedule="role_split",
                            align="words")
            assert q.wait_steady == (min(63, (S - 2) * 4 * per_tile) if S > 1 else 0)
            u = tp.plan_map(A, B, 1 << 20, "horner32", tile, S, 2)
            assert (u.schedule, u.threads) == (tp.Schedule.UNIFORM, threads - 64)
            assert (p.ring_bytes, p.grid, p.num_tiles) == (u.ring_bytes, u.grid, u.num_tiles)
    # residency counts the extra wave: tile 1024 has 5 waves per workgroup, 6 fit a CU
    p = tp.plan_map(A, B, 1 << 26, "scale2", 1024, 2, 2, schedule="role_split")
    assert p.resident_cap == 4
    p = tp.plan_map(A, B, 1 << 26, "scale2", 1024, 2, 2, resident_cap=6, schedule="role_split")
    assert p.resident_cap == 0        # 6 x 5 waves already fill 32 wave slots
    assert _status(tp.plan_map, A, B, 10, "scale2", 1024, 2, 2, tilepipe._NO_BUDGET, 0, 2) == 1
    assert _status(tp.plan_map, A, B, 10, "scale2", 1024, 2, 2, tilepipe._NO_BUDGET, 0, -1) == 1


# ------------------------------------------------------------------ 2-D map
def test_map_2d_plan_geometry_and_paths():
    p = tp.plan_map_2d(A, 1000, B, 1024, 100, 1000, "scale2", 4, 256, 2, 3)
    assert (p.tile_units, p.threads, p.lane_chunks, p.tiles_per_block) == (1024, 256, 1, 3)
    bands, boxes = -(-100 // 4), -(-1000 // 256)
    assert (p.num_tiles, p.grid) == (bands * boxes, bands * -(-boxes // 3))
    assert p.ring_bytes == 2 * 1024 * 4 and p.lds_bytes >= p.ring_bytes
    assert p.path == tp.Path.X4
    # the pages' rule: 16-byte aligned pointer and a stride of whole chunks
    w = dict(align="words")
    assert tp.plan_map_2d(A + 4, 1000, B, 1024, 100, 1000, **w).path == tp.Path.SCALAR_LOAD
    assert tp.plan_map_2d(A, 1002, B, 1024, 100, 1000, **w).path == tp.Path.SCALAR_LOAD   # stride
    assert tp.plan_map_2d(A, 1000, B, 1026, 100, 1000, **w).path == tp.Path.SCALAR_STORE
    assert tp.plan_map_2d(A, 1000, B, 1024, 100, 998, **w).path == tp.Path.SCALAR          # cols
    # realign (the default): only cols decides
    for src, ss, dst, ds in ((A + 4, 1000, B, 1024), (A, 1002, B, 1024), (A, 1000, B + 12, 1027)):
        assert tp.plan_map_2d(src, ss, dst, ds, 100, 1000).path == tp.Path.X4
        assert tp.plan_map_2d(src, ss, dst, ds, 100, 998).path == tp.Path.SCALAR
    assert tp.plan_map_2d(A, 1000, B, 1024, 100, 1000).head == 0
    assert _status(tp.plan_map_2d, A, 1000, B, 1024, 100, 1000, align=7) == 1
    for br, bc, threads, lanes in [(1, 256, 64, 1), (64, 4, 64, 1), (2, 4096, 256, 8), (16, 64, 256, 1)]:
        p = tp.plan_map_2d(A, 8192, B, 8192, 50, 5000, "copy", br, bc, 1, 1)
        assert (p.threads, p.lane_chunks) == (threads, lanes)
    # nothing to do: no launch, null pointers accepted
    assert tp.plan_map_2d(0, 0, 0, 0, 0, 10).grid == 0
    assert tp.plan_map_2d(0, 0, 0, 0, 10, 0).grid == 0


@pytest.mark.parametrize("args,status", [
    ((A, 100, B, 100, 10, 100, "scale2", 4, 2), 1),        # box_cols < 4
    ((A, 100, B, 100, 10, 100, "scale2", 0, 256), 1),      # only one side of the box given
    ((A, 100, B, 100, 10, 100, "scale2", 3, 256), 1),      # box_rows not a power of two
    ((A, 100, B, 100, 10, 100, "scale2", 4, 32), 1),       # box of 128 floats
    ((A, 100, B, 100, 10, 100, "scale2", 4, 4096), 1),     # box of 16384 floats
    ((A, 99, B, 100, 10, 100), 1),                         # stride < cols
    ((A, 100, B, 100, 10, 100, "nope"), 1),
    ((A, 100, B, 100, -1, 100), 1),
    ((A, 1 << 37, B, 100, 10, 100), 1),                    # stride too large
    ((A, 1 << 20, B, 100, 10, 100, "scale2", 512, 4), 1),  # a band spans more than 1 GiB
    ((A + 2, 100, B, 100, 10, 100), 2),
    ((A, 100, B + 1, 100, 10, 100), 2),
    ((A, 100, A + 400, 100, 10, 100), 4),                  # dst window inside src's range
    ((A, 100, A, 200, 10, 100), 4),                        # same base, other stride
    ((0, 100, B, 100, 10, 100), 1),
])
def test_map_2d_plan_errors(args, status):
    assert _status(tp.plan_map_2d, *args) == status


def test_map_2d_workgroup_windows_stay_inside_the_matrix():
    # Each workgroup of the 2-D kernel rebases its two buffer descriptors at its
    # band and run: base = r0 * stride + c0, num_records = ((rr - 1) * stride + cc) * 4,
    # with band = b / runs_per_band, r0 = band * box_rows, c0 = first box * box_cols.
    # Every access is range-checked against that window, so the window lying
    # inside the caller's matrix (and in 32 bits) bounds every access.
    for rows, cols, ss, br, bc, T in [(1, 1, 1, 1, 256, 2), (5, 3, 7, 64, 4, 1), (100, 1000, 1003, 4, 256, 3),
                                      (257, 64, 64, 16, 64, 2), (3, 9000, 9000, 1, 8192, 1),
                                      (1000, 5, 8, 2, 128, 65536), (37, 37, 40, 8, 32, 5)]:
        p = tp.plan_map_2d(A, ss, B, ss, rows, cols, "copy", br, bc, 1, T)
        runs = -(-(-(-cols // bc)) // p.tiles_per_block)
        extent = (rows - 1) * ss + cols
        assert p.grid == -(-rows // br) * runs
        for b in range(p.grid):
            band, first_box = b // runs, (b % runs) * p.tiles_per_block
            r0, c0 = band * br, first_box * bc
            rr, cc = min(br, rows - r0), min(p.tiles_per_block * bc, cols - c0)
            assert rr >= 1 and cc >= 1, (rows, cols, b)
            base, n = r0 * ss + c0, (rr - 1) * ss + cc
            assert 0 <= base and base + n <= extent and n * 4 < 1 << 32, (rows, cols, b)


def test_map_2d_default_box():
    # 0 x 0: 1024-float boxes, as wide as the window allows
    for cols, units in [(1, 1024), (4, 1024), (5, 1024), (300, 1024), (1024, 1024), (16384, 1024)]:
        assert tp.plan_map_2d(A, 20000, B, 20000, 10, cols).tile_units == units
    p = tp.plan_map_2d(A, 16448, B, 16384, 16384, 16384)
    assert p.grid == 16384 * (16 // 2)              # 1 x 1024 boxes, runs of 2
    p = tp.plan_map_2d(A, 64, B, 64, 1000, 64)
    assert p.grid == -(-1000 // 16)                 # 16 x 64 boxes: one run per band
    assert _status(tp.plan_map_2d, A, 100, B, 100, 10, 100, "scale2", 0, 256) == 1


def test_map_2d_plan_in_place_and_budget():
    assert tp.plan_map_2d(A, 100, A, 100, 10, 100).grid > 0          # exact aliasing is allowed
    assert _status(tp.plan_map_2d, A, 100, B, 100, 10, 100, "scale2", 4, 2048, 8, 0,
                   160 * KIB) == 3                                   # 8 x 32 KiB of ring
    p = tp.plan_map_2d(A, 100, B, 100, 10, 100, "horner32", 1, 256, 2, 2)
    assert (p.resident_cap, p.lds_bytes) == (0, p.ring_bytes)       # horner32: not bounded


# ------------------------------------------------- binding argument checks
def test_binding_rejects_bad_tensors_before_the_library():
    import torch
    x = torch.zeros(16)
    with pytest.raises(ValueError):
        tp.pipelined_map(x, x.clone())                         # a CPU tensor: no CPU path
    with pytest.raises(ValueError):
        tp.pipelined_map(x, x.clone(), "cube")                 # unknown op
    with pytest.raises(ValueError):
        tilepipe._schedule("eager")
    assert tilepipe._schedule("role_split") == tp.Schedule.ROLE_SPLIT
    assert tilepipe._schedule(7) == 7                          # passed through; the library decides
    with pytest.raises(TypeError):
        tp.map_2d(x.view(4, 4), x.view(4, 4).clone())         # not CUDA tensors
    with pytest.raises(ValueError):
        tp.map_2d(x.view(4, 4), x.view(2, 8), "cube")
    with pytest.raises(ValueError):
        tp.row_shift(x.view(4, 4))                             # a CPU tensor
    with pytest.raises(ValueError):
        tilepipe._row_stride(x.view(4, 4).t(), "src")          # column stride 4


# ------------------------------------------------------------ row shift
def test_row_shift_plan():
    p = tp.plan_row_shift(A, B, 64)
    assert (p.threads, p.grid, p.lds_bytes, p.path) == (64, 1, 1024, tp.Path.X4)
    p = tp.plan_row_shift(A, B, 65)
    assert (p.threads, p.lds_bytes) == (128, 2048)
    assert tp.plan_row_shift(A + 4, B, 3).path == tp.Path.SCALAR_LOAD
    assert tp.plan_row_shift(A, A, 1024).grid == 1
    assert tp.plan_row_shift(0, 0, 0).grid == 0
    assert _status(tp.plan_row_shift, A, B, 1025) == 1
    assert _status(tp.plan_row_shift, A, B, -1) == 1
    assert _status(tp.plan_row_shift, 0, B, 4) == 1
    assert _status(tp.plan_row_shift, A + 1, B, 4) == 2
    assert _status(tp.plan_row_shift, A, A + 16, 4) == 4


# ----------------------------------------------------------- chunk copy
def test_chunk_copy_plan():
    p = tp.plan_chunk_copy(A, B, 1 << 26, stages=2, tiles_per_block=64)
    assert (p.threads, p.tile_units, p.num_tiles, p.grid) == (256, 256, 1 << 18, 1 << 12)
    assert p.lds_bytes == 2 * 4096 + 3 * 3072
    assert p.wait_steady == 0 * 4 + 1 * 1
    # default: runs of one tile on the one-stage schedule
    p = tp.plan_chunk_copy(A, B, 1 << 26)
    assert (p.stages, p.tiles_per_block, p.grid, p.wait_steady) == (1, 1, 1 << 18, 0)
    assert p.lds_bytes == 4096 + 3072
    assert tp.plan_chunk_copy(A, B, 10, stages=4).wait_steady == 2 * 4 + 3 * 1
    assert tp.plan_chunk_copy(A + 4, B + 4, 10, stages=3).wait_steady == 1 * 7 + 2 * 4
    assert tp.plan_chunk_copy(A + 4, B, 10).path == tp.Path.SCALAR_LOAD
    assert tp.plan_chunk_copy(A, A, 10).grid == 1
    assert tp.plan_chunk_copy(0, 0, 0).grid == 0


def test_chunk_copy_ring_cut_to_the_run():
    # more slots than the run plus one hold nothing: the ring is cut to
    # tiles_per_block + 1 slots, and a run of one tile takes the one-stage
    # schedule (the same instructions in less LDS)
    for stages, tpb, eff in ((8, 2, 3), (8, 1, 1), (2, 1, 1), (4, 3, 4), (2, 5, 2), (5, 64, 5),
                             (3, 2, 3), (1, 7, 1)):
        p = tp.plan_chunk_copy(A, B, 100000, stages=stages, tiles_per_block=tpb)
        assert (p.stages, p.tiles_per_block) == (eff, tpb), (stages, tpb)
        assert p.lds_bytes == eff * 4096 + (2 * eff - 1) * 3072
    # the LDS budget is checked on the ring that runs
    assert tp.plan_chunk_copy(A, B, 10, stages=8, tiles_per_block=1,
                              lds_budget=8 * 1024).stages == 1


def test_chunk_copy_plan_errors():
    assert _status(tp.plan_chunk_copy, A, B, -1) == 1
    assert _status(tp.plan_chunk_copy, 0, B, 1) == 1
    assert _status(tp.plan_chunk_copy, A + 2, B, 1) == 2
    assert _status(tp.plan_chunk_copy, A, A + 16, 4) == 4
    # dst overlapping a metadata array
    assert _status(tp.plan_chunk_copy, A, B, 100, B + 50) == 4
    assert _status(tp.plan_chunk_copy, A, B, 100, 0, 0, B + 1599) == 4
    assert tp.plan_chunk_copy(A, B, 100, B + 1600, A, A).grid == 1   # metadata may alias src
    assert _status(tp.plan_chunk_copy, A, B, 1, 0, 0, 0, 9) == 1
    assert _status(tp.plan_chunk_copy, A, B, 1, 0, 0, 0, 8, 0, 8 * 4096) == 3


def test_chunk_copy_widths_plan():
    # 4- and 8-byte chunks move as words on both sides; the ring holds 256 chunks per slot
    for w, ld, st in ((4, 1, 1), (8, 2, 2), (16, 1, 1)):
        p = tp.plan_chunk_copy(A, B, 1000, stages=3, chunk_bytes=w)
        assert p.chunk_bytes == w and p.threads == 256
        assert p.path == (tp.Path.X4 if w == 16 else tp.Path.SCALAR)
        assert p.ring_bytes == 3 * 256 * w + 5 * 3 * 256 * 4
        assert p.wait_steady == 1 * (3 + ld) + 2 * st                      # (S-2) ld + (S-1) st
        assert (p.num_tiles, p.grid) == (4, 1 if w == 4 else 2)   # default runs 2, 2, 8
    assert tp.plan_chunk_copy(A + 4, B + 4, 10, chunk_bytes=8).path == tp.Path.SCALAR
    assert tp.plan_chunk_copy(A, B, 10).chunk_bytes == 16
    for bad in (0, 2, 12, 32):
        assert _status(tp.plan_chunk_copy, A, B, 10, chunk_bytes=bad) == 1
    # overlap is judged on n x chunk_bytes bytes
    assert tp.plan_chunk_copy(A, A + 400, 100, chunk_bytes=4).grid == 1
    assert _status(tp.plan_chunk_copy, A, A + 400, 101, chunk_bytes=4) == 4


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(16)
    with pytest.raises(ValueError):
        tp.pipelined_map(x, x.clone())
    with pytest.raises(ValueError):
        tp.row_shift(x.reshape(4, 4))
    with pytest.raises(ValueError):
        tp.chunk_copy(torch.zeros(16, dtype=torch.uint8), torch.zeros(16, dtype=torch.uint8))
    with pytest.raises(ValueError):
        tp.pipelined_map(x, x.clone(), op="bogus")


def test_header_is_plain_c():
    # the ABI header must compile as C without HIP headers
    import subprocess
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "t.c")
        fields = [f for f, _ in tilepipe._CPlan._fields_]
        with open(src, "w") as f:
            f.write('#include <stddef.h>\n#include <stdio.h>\n#include "tilepipe.h"\n'
                    'int main(void){printf("%zu", sizeof(tp_plan));'
                    + "".join(f'printf(" %zu", offsetof(tp_plan, {n}));' for n in fields)
                    + "return TP_OK;}\n")
        exe = os.path.join(d, "t")
        subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", f"-I{ROOT}/include", src, "-o", exe],
                       check=True)
        # the binding's mirror of tp_plan has the C struct's size and offsets
        got = [int(v) for v in subprocess.run([exe], capture_output=True, text=True).stdout.split()]
        assert got[0] == ctypes.sizeof(tilepipe._CPlan)
        assert got[1:] == [getattr(tilepipe._CPlan, n).offset for n in fields]


# ------------------------------------------------------- copies between workgroups
def test_workgroup_copy_plan():
    n = 1000
    need = tp.workgroup_copy_workspace_bytes(n)
    assert need == 512 * n                  # 64 tagged 8-byte words per chunk
    W, S = 0x7f8000000000, 0x7fc000000000
    p = tp.plan_workgroup_copy(A, B, n, W, need, S)
    assert (p.grid, p.threads, p.lds_bytes, p.tile_units) == (n, 64, 512, 256)
    assert tp.plan_workgroup_copy(A, A, n, W, need, S).grid == n              # in place
    assert tp.plan_workgroup_copy(0, 0, 0, 0, 0, 0).grid == 0                 # nothing to do
    assert tp.workgroup_copy_workspace_bytes(0) == 0
    with pytest.raises(ValueError):
        tp.workgroup_copy_workspace_bytes(-1)


def test_workgroup_copy_plan_errors():
    n = 1000
    need = tp.workgroup_copy_workspace_bytes(n)
    W, S = 0x7f8000000000, 0x7fc000000000
    f = tp.plan_workgroup_copy
    assert _status(f, A, B, n, W, need - 1, S) == 1          # short workspace
    assert _status(f, A, B, n, 0, need, S) == 1              # no workspace
    assert _status(f, A, B, n, W, need, 0) == 1              # no status word
    assert _status(f, A, B, -1, W, need, S) == 1
    assert _status(f, A, B, (1 << 26) + 1, W, 1 << 40, S) == 1
    assert _status(f, A, B, n, W, need, S, -1) == 1          # spin limit
    assert _status(f, A, B, n, W, need, S, (1 << 24) + 1) == 1
    assert _status(f, A + 2, B, n, W, need, S) == 2
    assert _status(f, A, B, n, W + 2, need, S) == 2
    assert _status(f, A, B, n, W + 4, need, S) == 2          # tagged words need 8-byte alignment
    assert _status(f, A, B, n, W, need, S + 2) == 2
    assert _status(f, A, A + 256, n, W, need, S) == 4        # dst overlapping src in part
    assert _status(f, A, B, n, B + 256, need, S) == 4        # workspace inside dst
    assert _status(f, A, B, n, W, need, A + 8) == 4          # status inside src
    assert _status(f, A, B, n, W, need, W + need - 4) == 4   # status inside the workspace
