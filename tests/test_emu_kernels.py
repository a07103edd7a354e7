"""The pipelined map (both schedules), the 2-D map and the row exchange under
the CPU emulator (tests/emu): the same kernel-body source the gfx950 kernels
are built from, planned by the library's planner, run in wave lock-step with
every access checked against the caller's buffers, every LDS read against the
wait that retires its load, LDS shared between waves against the barriers,
and no load in flight when a wave ends. Results must equal the oracle bit for
bit ("Asynchronous Data Movement", section "Double buffering"; "Asynchronous
Copies", section "A Global-to-Shared Copy").

These kernels also pass their parity tests on the GPU; here the emulator
reaches launches of the full workload sizes (sampled workgroups) and the
stage/lane-chunk/path matrix without a GPU, and the last tests plant mistakes
that it must report. Policies 2 and 3 leave random bytes, instead of zeros,
in the LDS slots of lanes whose loads fail the range check."""
import numpy as np
import pytest

import oracle
from tests import emu


@pytest.fixture(scope="module", autouse=True)
def _built():
    emu.build()


def _floats(n, seed, offset_words=0, line=128):
    """n floats in [-1, 1) whose address is offset_words words past a
    `line`-byte boundary."""
    raw = np.zeros(n + line // 4 + 64, np.float32)
    start = ((-raw.ctypes.data) % line) // 4 + offset_words
    a = raw[start:start + n]
    a[:] = (np.random.default_rng(seed).random(n, dtype=np.float32) * 2 - 1)
    return a


def _out(n, offset_words=0, line=128):
    raw = np.full(n + line // 4 + 64, np.nan, np.float32)
    start = ((-raw.ctypes.data) % line) // 4 + offset_words
    return raw[start:start + n]


def _bits(a):
    return a.view(np.uint32)


def _map_case(n, op, tile, stages, tpb, in_off=0, out_off=0, align="realign", schedule="uniform",
              policy=0, seed=0, lds_base=0, resident_cap=0):
    x = _floats(n, seed=n + tile + stages, offset_words=in_off)
    y = _out(n, out_off)
    plan = emu.pipelined_map(x, y, op, tile, stages, tpb, resident_cap=resident_cap,
                             schedule=schedule, align=align, policy=policy, seed=seed,
                             lds_base=lds_base)
    what = (f"n={n} op={op} tile={tile} S={stages} T={tpb} in+{in_off} out+{out_off} {align} "
            f"{schedule} path={plan.path} head={plan.head} policy={policy}")
    assert np.array_equal(_bits(y), _bits(oracle.pipelined_map(x, op))), what
    return plan


# ------------------------------------------------------------------ 1-D map
@pytest.mark.parametrize("tile", [256, 512, 1024, 2048, 4096, 8192])
def test_map_stages_and_tiles(tile):
    # several workgroups, a ragged tail and runs of 1-3 tiles at every stage count
    n = 3 * tile * 3 + 37
    for stages in range(1, min(8, (160 * 1024 - 256) // (4 * tile)) + 1):
        for tpb in (1, 3):
            _map_case(n, "scale2", tile, stages, tpb, policy=(stages + tpb) % 4, seed=stages,
                      lds_base=1024 * (tpb == 3))


@pytest.mark.parametrize("align", ["realign", "words"])
def test_map_offsets_and_paths(align):
    # in and out at every word offset from a line; the pages' 4-byte paths
    # under "words", the 128-byte realignment (head of 0-31 floats) otherwise
    seen = set()
    for in_off in range(0, 32, 5):
        for out_off in (0, 1, 2, 3, 17, 31):
            for stages in (1, 2, 3):
                plan = _map_case(2 * 1024 + 300 + in_off, "scale2", 1024, stages, 2, in_off,
                                 out_off, align=align, policy=(stages + in_off) % 4, seed=in_off)
                seen.add(plan.path)
    assert seen == ({0} if align == "realign" else {0, 1, 2, 3})


def test_map_small_and_edge_sizes():
    for n in (1, 2, 3, 4, 5, 31, 32, 33, 63, 64, 65, 255, 257):
        for out_off in (0, 3, 31):
            _map_case(n, "scale2", 256, 2, 2, 1, out_off, policy=n % 2)


def test_map_ops():
    for stages in (1, 2, 4):
        for tile in (256, 1024, 2048):
            _map_case(2 * tile * 2 + 13, "horner32", tile, stages, 2, 0, 3, policy=stages % 2)
    for align, offs in (("realign", (1, 2)), ("words", (0, 0)), ("words", (1, 0)), ("words", (0, 1)),
                        ("words", (1, 1))):
        _map_case(4 * 1024 + 9, "copy", 1024, 2, 2, *offs, align=align)


def test_map_residency_bound_and_in_place():
    for cap in (-1, 0, 1, 5, 17):
        _map_case(5 * 256 + 3, "scale2", 256, 2, 2, resident_cap=cap)
    x = _floats(3 * 1024 + 11, seed=9, offset_words=2)
    expected = oracle.pipelined_map(x, "horner32")
    for stages in (1, 2, 4):
        y = _out(x.size, 2)
        y[:] = x
        emu.pipelined_map(y, y, "horner32", 1024, stages, 2, policy=stages % 2)
        assert np.array_equal(_bits(y), _bits(expected)), stages


def test_role_split_schedule():
    for stages in range(1, 9):
        for tile in (256, 1024, 8192):
            if stages * tile * 4 + 256 > 160 * 1024:
                continue
            _map_case(2 * tile * 3 + 21, "scale2", tile, stages, 3, schedule="role_split",
                      policy=stages % 4, seed=stages)
    for in_off, out_off in ((1, 0), (0, 1), (1, 1)):
        _map_case(3 * 1024 + 5, "scale2", 1024, 2, 2, in_off, out_off, align="words",
                  schedule="role_split")
    for stages in (1, 2, 4):
        _map_case(3 * 1024 + 5, "horner32", 1024, stages, 2, schedule="role_split")


def test_full_size_map_launches():
    # the step (2^28 floats, tile 256, 2 stages, runs of 4: 262144 workgroups)
    # and the 4-byte-offset sweep point, on full-size buffers whose untouched
    # pages are never allocated: the first workgroups, one in the middle and
    # the last ones run
    n = 1 << 28
    for in_off in (0, 1):
        xraw = np.zeros(n + 64, np.float32)
        yraw = np.zeros(n + 64, np.float32)
        xs = ((-xraw.ctypes.data) % 128) // 4
        ys = ((-yraw.ctypes.data) % 128) // 4
        x = xraw[xs + in_off:xs + in_off + n]
        y = yraw[ys:ys + n]
        plan = emu.pipelined_map(x, y, "scale2", 256, 2, 0, blocks=[0], regions=[(x, False), (y, True)])
        last = plan.grid - 1
        blocks = [0, 1, plan.grid // 2, last - 1, last]
        per = plan.tiles_per_block * 256
        for b in blocks:
            lo = max(0, b * per - 32)
            hi = min(n, (b + 1) * per + 32)
            x[lo:hi] = np.random.default_rng(b).random(hi - lo, dtype=np.float32) * 2 - 1
        plan = emu.pipelined_map(x, y, "scale2", 256, 2, 0, blocks=blocks,
                                 regions=[(x, False), (y, True)], policy=in_off)
        assert plan.tiles_per_block == 4
        assert plan.grid == (262144 if in_off == 0 else plan.grid)
        for b in blocks:
            lo = plan.head + b * per
            hi = min(n, plan.head + (b + 1) * per)
            if b == last:
                hi = n
            if b == 0:
                lo = 0
            assert np.array_equal(_bits(y[lo:hi]), _bits(x[lo:hi] * np.float32(2))), (in_off, b)
        del xraw, yraw


def test_map_past_4_gib():
    # 2^30 + 7 floats (a 4 GiB + 28 B buffer): the workgroups around the 4 GiB
    # byte boundary and the last one with its ragged end
    n = (1 << 30) + 7
    x = np.zeros(n, np.float32)
    y = np.zeros(n, np.float32)
    plan = emu.pipelined_map(x, y, "scale2", 1024, 2, 2, blocks=[0])
    per = 2 * 1024
    b4 = ((1 << 30) - plan.head) // per
    blocks = [b4 - 1, b4, plan.grid - 1]
    for b in blocks:
        lo, hi = max(0, plan.head + b * per - 8), min(n, plan.head + (b + 1) * per + 8)
        x[lo:hi] = np.random.default_rng(b).random(hi - lo, dtype=np.float32) * 2 - 1
    emu.pipelined_map(x, y, "scale2", 1024, 2, 2, blocks=blocks, policy=1)
    for b in blocks:
        lo, hi = plan.head + b * per, min(n, plan.head + (b + 1) * per)
        if b == plan.grid - 1:
            hi = n
        assert np.array_equal(_bits(y[lo:hi]), _bits(x[lo:hi] * np.float32(2))), b


# ------------------------------------------------------------------ 2-D map
def _matrix(rows, stride, seed, offset_words=0):
    raw = np.zeros(rows * stride + 64, np.float32)
    start = ((-raw.ctypes.data) % 128) // 4 + offset_words
    m = raw[start:start + rows * stride].reshape(rows, stride)
    m[:] = np.random.default_rng(seed).random(m.shape, dtype=np.float32) * 2 - 1
    return raw, m


def _map2d_case(rows, cols, ss, ds, op, box, stages, tpb, offs=(0, 0), align="realign", policy=0):
    sraw, sm = _matrix(rows, ss, seed=rows * cols + ss, offset_words=offs[0])
    draw, dm = _matrix(rows, ds, seed=ds, offset_words=offs[1])
    src, dst = sm[:, :cols], dm[:, :cols]
    expected = dm.copy()
    oracle.map_2d(src, expected[:, :cols], op)
    plan = emu.map_2d(src, dst, op, box[0], box[1], stages, tpb, align=align, policy=policy,
                      src_region=(sraw, False), dst_region=(draw, True))
    what = f"{rows}x{cols} ss={ss} ds={ds} {op} box={box} S={stages} T={tpb} offs={offs} {align}"
    assert np.array_equal(_bits(dm), _bits(expected)), what   # the gaps between rows too
    return plan


@pytest.mark.parametrize("shape", [(1, 4), (5, 300), (37, 300), (64, 1024), (130, 77), (3, 2049)])
def test_map_2d_shapes_boxes_stages(shape):
    rows, cols = shape
    for box in ((0, 0), (1, 256), (4, 64), (16, 16), (2, 512)):
        for stages in (1, 2, 3, 5, 8):
            ss = cols + (8 if stages % 2 else 5)
            _map2d_case(rows, cols, ss, cols + 4 * (stages % 3), "scale2", box, stages,
                        1 + stages % 3, policy=stages % 4)


def test_map_2d_paths_and_ops():
    # under "words" a side takes 4-byte accesses unless its pointer is 16-byte
    # aligned and its row stride a multiple of 4 floats; "realign" keeps
    # 16-byte accesses whenever cols is a multiple of 4
    seen = set()
    for offs, ss, ds in (((0, 0), 204, 200), ((1, 0), 204, 200), ((0, 2), 204, 200),
                         ((0, 0), 203, 201), ((3, 1), 205, 202)):
        for align in ("realign", "words"):
            plan = _map2d_case(21, 200, ss, ds, "scale2", (4, 64), 2, 2, offs, align)
            seen.add((align, plan.path))
    assert seen == {("realign", 0), ("words", 0), ("words", 1), ("words", 2), ("words", 3)}
    _map2d_case(19, 300, 304, 300, "horner32", (4, 256), 2, 2)
    _map2d_case(19, 301, 305, 303, "horner32", (4, 256), 2, 2, align="words")
    _map2d_case(19, 300, 308, 300, "copy", (4, 256), 2, 2)


def test_map_2d_full_size_edges():
    # the 2-D workload: a 16384 x 16384 window of a matrix whose rows are
    # 16448 floats apart, into a dense matrix, boxes 1 x 1024, 2 stages, runs
    # of 2 (8 runs per band, 131072 workgroups): the first and last runs of
    # the first and last bands
    R, C, SS = 16384, 16384, 16448
    sraw = np.zeros(R * SS, np.float32)
    draw = np.zeros(R * C, np.float32)
    sm, dm = sraw.reshape(R, SS), draw.reshape(R, C)
    plan = emu.map_2d(sm[:, :C], dm, "scale2", 1, 1024, 2, 2, blocks=[0],
                      src_region=(sraw, False), dst_region=(draw, True))
    runs = plan.grid // R
    blocks = [0, runs - 1, plan.grid - runs, plan.grid - 1]
    for b in blocks:
        r, c0 = b // runs, (b % runs) * 2048
        sm[r, c0:c0 + 2048] = np.random.default_rng(b).random(2048, dtype=np.float32) * 2 - 1
    emu.map_2d(sm[:, :C], dm, "scale2", 1, 1024, 2, 2, blocks=blocks, policy=1,
               src_region=(sraw, False), dst_region=(draw, True))
    for b in blocks:
        r, c0 = b // runs, (b % runs) * 2048
        assert np.array_equal(_bits(dm[r, c0:c0 + 2048]), _bits(sm[r, c0:c0 + 2048] * np.float32(2)))


# ------------------------------------------------------------- row exchange
@pytest.mark.parametrize("rows", [1, 2, 63, 64, 65, 200, 1000, 1024])
def test_row_shift(rows):
    for a_off, b_off in ((0, 0), (1, 0), (0, 3)):
        araw = np.zeros(rows * 4 + 64, np.float32)
        s = ((-araw.ctypes.data) % 64) // 4 + a_off
        a = araw[s:s + rows * 4].reshape(rows, 4)
        a[:] = np.random.default_rng(rows).random((rows, 4), dtype=np.float32)
        b = _out(rows * 4, b_off).reshape(rows, 4)
        emu.row_shift(a, b, policy=(rows + a_off) % 4, seed=a_off)
        assert np.array_equal(_bits(b), _bits(oracle.row_shift(a))), (rows, a_off, b_off)
    # in place: the whole input is in LDS before anything is written
    c = a.copy()
    emu.row_shift(c, c)
    assert np.array_equal(_bits(c), _bits(oracle.row_shift(a)))


# ----------------------------------------------------------- planted mistakes
@pytest.mark.parametrize("case", ["wave_local", "barrier", "role_split", "map_2d", "row_shift"])
def test_planted_short_wait_is_reported(case):
    x = _floats(3 * 1024 + 8, seed=1)
    y = _out(x.size)
    with pytest.raises(emu.EmulationError):
        if case == "wave_local":
            emu.pipelined_map(x, y, "scale2", 1024, 3, 2, wait_bias=1)
        elif case == "barrier":
            emu.pipelined_map(x, _out(x.size, 1), "scale2", 1024, 3, 2, align="words", wait_bias=1)
        elif case == "role_split":
            emu.pipelined_map(x, y, "scale2", 1024, 3, 2, schedule="role_split", wait_bias=1)
        elif case == "map_2d":
            emu.map_2d(x[:3072].reshape(3, 1024), y[:3072].reshape(3, 1024), "scale2", 1, 1024, 2, 2,
                       wait_bias=1)
        else:
            emu.row_shift(x[:256].reshape(64, 4), y[:256].reshape(64, 4), wait_bias=1)


@pytest.mark.parametrize("case", ["barrier", "role_split", "row_shift"])
def test_planted_missing_barriers_are_reported(case):
    # the schedules whose lanes read bytes other waves loaded: without their
    # barriers, a wave reads LDS another wave wrote (or reloads LDS another
    # wave still reads) with nothing ordering the two
    x = _floats(3 * 1024 + 8, seed=3)
    drop = 4
    with pytest.raises(emu.EmulationError, match="no barrier|no load of this workgroup wrote"):
        if case == "barrier":
            emu.pipelined_map(x, _out(x.size, 1), "scale2", 1024, 2, 2, align="words", policy=drop)
        elif case == "role_split":
            emu.pipelined_map(x, _out(x.size), "scale2", 1024, 2, 2, schedule="role_split",
                              policy=drop)
        else:
            emu.row_shift(x[:512].reshape(128, 4), _out(512).reshape(128, 4), policy=drop)


def test_planted_short_buffers_are_reported():
    x = _floats(2 * 1024, seed=2)
    y = _out(x.size)
    with pytest.raises(emu.EmulationError, match="reads outside every buffer"):
        emu.pipelined_map(x, y, "scale2", 1024, 2, 2, regions=[(x[:-4], False), (y, True)])
    with pytest.raises(emu.EmulationError, match="outside every writable buffer"):
        emu.pipelined_map(x, y, "scale2", 1024, 2, 2, regions=[(x, False), (y[:-1], True)])
