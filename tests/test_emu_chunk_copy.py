"""The chunk copy's kernel body under the CPU emulator (tests/emu): the same
source the gfx950 kernels are built from, planned by the library's planner,
run lane by lane in wave lock-step. Each case must match the oracle bit for
bit under both landing policies, with every access inside the caller's
buffers, every LDS read after the wait that retires its load, and no load in
flight when a wave ends ("Asynchronous Copies", section "A Global-to-Shared
Copy", the paragraph on the copy's operands).

Policies 2 and 3 also leave random bytes, instead of zeros, in the LDS slots
of lanes whose loads fail the range check: no result may depend on them.

The last tests plant mistakes in what the emulator is given (a wait count one
too small, buffers registered one chunk short) and require it to report them."""
import numpy as np
import pytest
import torch

import oracle
from software_pipelining_amd import workloads
from tests import emu

DEADBEEF = 0xDEADBEEF


@pytest.fixture(scope="module", autouse=True)
def _built():
    emu.build()


def _at(nbytes, offset_words, fill=None):
    """A uint8 array of nbytes whose address is offset_words words past a
    64-byte boundary."""
    raw = np.zeros(nbytes + 128, np.uint8)
    start = (-raw.ctypes.data) % 64 + 4 * offset_words
    a = raw[start:start + nbytes]
    if fill is not None:
        a[:] = fill
    return a


def _inputs(inp, src_off=0, dst_off=0, chunk_bytes=16):
    src = _at(inp.src.numel(), src_off, inp.src.numpy().reshape(-1))
    dst = _at(inp.dst_init.numel(), dst_off, inp.dst_init.numpy().reshape(-1))
    meta = [m.numpy().copy() for m in (inp.pred, inp.src_size, inp.ignore_src)]
    return src, dst, meta


def _check(inp, stages, tpb=0, src_off=0, dst_off=0, use=(True, True, True), policy=0, seed=0,
           chunk_bytes=16):
    src, dst, meta = _inputs(inp, src_off, dst_off)
    meta = [m if u else None for m, u in zip(meta, use)]
    expected = oracle.chunk_copy(src, dst, *meta, chunk_bytes=chunk_bytes)
    plan = emu.chunk_copy(src, dst, *meta, chunk_bytes=chunk_bytes, stages=stages,
                          tiles_per_block=tpb, policy=policy, seed=seed)
    what = f"n={src.size // chunk_bytes} W={chunk_bytes} S={stages} T={tpb} path={plan.path} " \
           f"offsets={src_off},{dst_off} use={use} policy={policy}"
    assert np.array_equal(dst, expected), what
    return plan


def _combos_inputs():
    pred_vals = [0, 1, 7, 255]
    ign_vals = [0, 1, 200]
    size_vals = list(range(17)) + [17, 100, 255]
    combos = [(p, g, s) for p in pred_vals for g in ign_vals for s in size_vals]
    n = len(combos)
    g = torch.Generator().manual_seed(3)
    return workloads.ChunkCopyInputs(
        src=torch.randint(1, 256, (n, 16), generator=g, dtype=torch.int64).to(torch.uint8),
        dst_init=workloads.prefill_words(n * 4).view(torch.uint8).reshape(n, 16),
        pred=torch.tensor([c[0] for c in combos], dtype=torch.uint8),
        src_size=torch.tensor([c[2] for c in combos], dtype=torch.uint8),
        ignore_src=torch.tensor([c[1] for c in combos], dtype=torch.uint8))


@pytest.mark.parametrize("policy", [0, 1, 2, 3])
def test_operand_combinations_all_paths(policy):
    inp = _combos_inputs()
    for stages in (1, 2, 3):
        for src_off, dst_off in ((0, 0), (1, 0), (0, 1), (2, 3)):
            plan = _check(inp, stages, 0, src_off, dst_off, policy=policy, seed=stages)
            assert plan.path == (1 if src_off % 4 else 0) | (2 if dst_off % 4 else 0)


@pytest.mark.parametrize("n", [1, 3, 255, 256, 257, 1000, 64 * 256 + 1, 3 * 64 * 256 + 100])
def test_sizes_and_stages(n):
    inp = workloads.chunk_copy_inputs(n, seed=n)
    stage_list = range(1, 9) if n <= 1000 else (1, 2, 4, 8)
    for stages in stage_list:
        off = (0, 0) if stages % 2 else (3, 2)
        _check(inp, stages, 0, *off, policy=stages % 4, seed=stages)


def test_tiles_per_block():
    inp = workloads.chunk_copy_inputs(3 * 256 + 5, seed=11)
    for tpb in (1, 2, 3, 7, 1000):
        for stages in (1, 2, 4):
            _check(inp, stages, tpb, policy=tpb % 2)


@pytest.mark.parametrize("use", [(False, False, False), (True, False, False), (False, True, False),
                                 (False, False, True), (True, True, False), (False, True, True),
                                 (True, False, True)])
def test_absent_metadata(use):
    inp = workloads.chunk_copy_inputs(2 * 256 + 17, seed=12, sizes=tuple(range(18)), p_ignore=0.2)
    for stages in (1, 3):
        _check(inp, stages, 0, use=use, policy=stages % 2)


def test_in_place():
    inp = workloads.chunk_copy_inputs(4 * 256 + 9, seed=13)
    for stages in (1, 2, 4):
        for policy in (0, 1):
            buf = _at(inp.src.numel(), 0, inp.src.numpy().reshape(-1))
            meta = [m.numpy().copy() for m in (inp.pred, inp.src_size, inp.ignore_src)]
            expected = oracle.chunk_copy(buf, buf, *meta)
            emu.chunk_copy(buf, buf, *meta, stages=stages, policy=policy,
                           regions=[(buf, True)] + [(m, False) for m in meta])
            assert np.array_equal(buf, expected)


@pytest.mark.parametrize("width", [4, 8])
def test_narrow_chunks(width):
    n = 3 * 256 + 7
    g = torch.Generator().manual_seed(width)
    src_t = torch.randint(0, 256, (n * width,), generator=g, dtype=torch.int64).to(torch.uint8)
    pred = (torch.rand(n, generator=g) < 0.8).to(torch.uint8).numpy()
    size = torch.randint(0, width + 3, (n,), generator=g, dtype=torch.int64).to(torch.uint8).numpy()
    ign = (torch.rand(n, generator=g) < 0.1).to(torch.uint8).numpy()
    for stages in (1, 2, 3, 4):
        for src_off, dst_off in ((0, 0), (1, 3)):
            src = _at(n * width, src_off, src_t.numpy())
            dst = _at(n * width, dst_off, np.frombuffer(
                np.full(n * width // 4, DEADBEEF, np.uint32).tobytes(), np.uint8))
            expected = oracle.chunk_copy(src, dst, pred, size, ign, chunk_bytes=width)
            emu.chunk_copy(src, dst, pred, size, ign, chunk_bytes=width, stages=stages,
                           policy=stages % 2)
            assert np.array_equal(dst, expected), (width, stages, src_off, dst_off)


@pytest.mark.parametrize("stages,tpb", [(1, 0), (2, 0), (3, 0), (4, 0), (2, 2), (2, 8), (2, 64)])
def test_full_size_boundary_workgroups(stages, tpb):
    # the chunk-copy workload's launches (2^26 chunks; the default runs of
    # max(1, S-1) tiles, and runs of 2, 8 and 64 tiles): the first, a middle
    # and the last workgroup run on buffers of the full size (pages that are
    # never touched are never allocated); only their ranges hold data
    n = 1 << 26
    run = tpb or max(1, stages - 1)
    per_block = run * 256
    grid = -(-n // per_block)                  # a run of 3 tiles leaves a short last run
    blocks = [0, grid // 2 - 1, grid - 1]
    rng = np.random.default_rng(5)
    src = np.zeros(n * 16, np.uint8)
    pred, size, ign = (np.zeros(n, np.uint8) for _ in range(3))
    for b in blocks:
        lo, hi = b * per_block, min(n, (b + 1) * per_block)
        src[16 * lo:16 * hi] = rng.integers(0, 256, 16 * (hi - lo), dtype=np.uint8)
        pred[lo:hi] = rng.random(hi - lo) < 0.9
        size[lo:hi] = rng.choice(np.array([0, 4, 8, 12, 16], np.uint8), hi - lo)
        ign[lo:hi] = rng.random(hi - lo) < 0.01
    fill = np.frombuffer(np.full(4 * per_block, DEADBEEF, np.uint32).tobytes(), np.uint8)
    dst = np.zeros(n * 16, np.uint8)
    for b in blocks:
        lo, hi = b * per_block, min(n, (b + 1) * per_block)
        dst[16 * lo:16 * hi] = fill[:16 * (hi - lo)]
    plan = emu.chunk_copy(src, dst, pred, size, ign, stages=stages, tiles_per_block=tpb,
                          blocks=blocks, policy=stages % 4)
    assert plan.grid == grid and plan.tiles_per_block == run
    for b in blocks:
        lo, hi = b * per_block, min(n, (b + 1) * per_block)
        exp = oracle.chunk_copy(src[16 * lo:16 * hi], fill[:16 * (hi - lo)], pred[lo:hi],
                                size[lo:hi], ign[lo:hi])
        assert np.array_equal(dst[16 * lo:16 * hi], exp), (stages, tpb, b)


def test_empty_launches_nothing():
    src = _at(0, 0)
    dst = _at(0, 0)
    plan = emu.chunk_copy(src, dst, None, None, None, stages=2)
    assert plan.grid == 0


# ----------------------------------------------------------- planted mistakes
@pytest.mark.parametrize("stages", [1, 2, 3, 4])
def test_planted_short_wait_is_reported(stages):
    inp = workloads.chunk_copy_inputs(2 * 256, seed=7)
    src, dst, meta = _inputs(inp)
    with pytest.raises(emu.EmulationError, match="still in flight"):
        emu.chunk_copy(src, dst, *meta, stages=stages, wait_bias=1)


def test_planted_short_destination_is_reported():
    inp = workloads.chunk_copy_inputs(300, seed=8, p_pred=1.0)
    src, dst, meta = _inputs(inp)
    regions = [(src, False), (dst[:-16], True)] + [(m, False) for m in meta]
    with pytest.raises(emu.EmulationError, match="outside every writable buffer"):
        emu.chunk_copy(src, dst, *meta, stages=2, regions=regions)


def test_planted_short_source_is_reported():
    inp = workloads.chunk_copy_inputs(300, seed=9, p_pred=1.0, p_ignore=0.0, sizes=(16,))
    src, dst, meta = _inputs(inp)
    regions = [(src[:-16], False), (dst, True)] + [(m, False) for m in meta]
    with pytest.raises(emu.EmulationError, match="reads outside every buffer"):
        emu.chunk_copy(src, dst, *meta, stages=3, regions=regions)


def test_random_configurations():
    # sizes, stages, runs, chunk widths, offsets, metadata presence and value
    # mixes drawn jointly
    rng = np.random.default_rng(17)
    for i in range(60):
        width = int(rng.choice([16, 16, 8, 4]))
        n = int(rng.choice([rng.integers(1, 300), rng.integers(1, 3000), rng.integers(1, 20000)]))
        stages = int(rng.integers(1, 9))
        tpb = int(rng.choice([0, 1, 2, 5, 64]))
        src_off, dst_off = (int(rng.integers(0, 4)), int(rng.integers(0, 4)))
        use = tuple(bool(rng.random() < 0.8) for _ in range(3))
        src = _at(n * width, src_off, rng.integers(0, 256, n * width, dtype=np.uint8))
        dst = _at(n * width, dst_off, rng.integers(0, 256, n * width, dtype=np.uint8))
        meta = [rng.integers(0, 2, n, dtype=np.uint8) * rng.integers(1, 256, n, dtype=np.uint8),
                rng.integers(0, width + 4, n, dtype=np.uint8),
                (rng.random(n) < rng.choice([0.0, 0.05, 0.5])).astype(np.uint8)]
        meta = [m if u else None for m, u in zip(meta, use)]
        expected = oracle.chunk_copy(src, dst, *meta, chunk_bytes=width)
        plan = emu.chunk_copy(src, dst, *meta, chunk_bytes=width, stages=stages,
                              tiles_per_block=tpb, policy=i % 4, seed=i)
        assert np.array_equal(dst, expected), (i, width, n, stages, tpb, src_off, dst_off, use,
                                               plan.path)


def test_device_check_accepts_only_gfx950():
    # the library's check of a device's architecture name: gfx950 with or
    # without feature suffixes passes, any other name is TP_ERR_UNSUPPORTED_DEVICE
    import ctypes
    f = emu.lib().emu_arch_status
    f.argtypes = [ctypes.c_char_p]
    f.restype = ctypes.c_int
    for name in (b"gfx950", b"gfx950:sramecc+:xnack-", b"gfx950:xnack+"):
        assert f(name) == 0, name
    for name in (b"gfx942", b"gfx942:sramecc+:xnack-", b"gfx9500", b"gfx95", b"gfx90a", b"",
                 b"gfx1100", b"sm_90"):
        assert f(name) == 5, name
    assert f(None) == 5
