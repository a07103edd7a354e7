"""GPU parity of tp_pipelined_map against the oracle (bit-exact), through the C
ABI, over stage counts, tile sizes, tiles per workgroup, both alignment
policies (16-byte accesses realigned to the output, and the pages' 4-byte
fallback with all four load/store paths), ragged sizes and in-place use.
Results must not depend on any of the performance parameters ("Asynchronous
Data Movement", sections "Double buffering" and "Alignment requirements")."""
import numpy as np
import pytest
import torch

import oracle
import software_pipelining_amd as tp
from software_pipelining_amd import workloads
from tests.gpu_util import assert_bits_equal, out_buffer, to_device

pytestmark = pytest.mark.gpu

OPS = ["scale2", "horner32", "copy"]
# empty, tail-only, sub-tile, tile edges, several tiles and workgroups with ragged ends
SIZES = [0, 1, 3, 4, 5, 63, 64, 255, 256, 257, 1023, 1024, 1029, 4099, 3 * 8192 + 5,
         64 * 1024 + 7, 2 * 64 * 1024 + 8]
TILES = [256, 512, 1024, 2048, 4096, 8192]
STAGES = [1, 2, 3, 4, 5, 8]
# float offsets of in / out from a 256-byte boundary; out offsets 0, 2, 1, 3, 4
# give realigned heads of 0, 30, 31, 29, 28 floats
PATH_OFFSETS = [(0, 0), (1, 0), (0, 2), (3, 1), (2, 3), (4, 4)]
ALIGNS = ["realign", "words"]


def _expected_path(in_off, out_off, align="realign"):
    if align == "realign":
        return tp.Path.X4
    return (tp.Path.SCALAR_LOAD if in_off % 4 else 0) | (tp.Path.SCALAR_STORE if out_off % 4 else 0)


def _run_case(dev, op, x_host, expected, in_off, out_off, tile, stages, tpb, budget,
              schedule="uniform", align="realign"):
    n = x_host.numel()
    x = to_device(x_host, dev, offset_words=in_off)
    y = out_buffer(n, torch.float32, dev, offset_words=out_off)
    kw = dict(schedule=schedule, align=align)
    plan = tp.plan_map(x.tensor.data_ptr(), y.tensor.data_ptr(), n, op, tile, stages, tpb, **kw)
    if plan.ring_bytes > budget and n > 0:     # an empty call launches nothing, so it succeeds
        with pytest.raises(tp.TilepipeError) as e:
            tp.pipelined_map(x.tensor, y.tensor, op, tile, stages, tpb, **kw)
        assert e.value.status == 3
        return False
    path = tp.pipelined_map(x.tensor, y.tensor, op, tile, stages, tpb, **kw)
    if n:
        assert path == _expected_path(in_off, out_off, align)
    what = (f"{op} {schedule} {align} n={n} in+{in_off} out+{out_off} tile={tile} S={stages} "
            f"T={tpb} path={int(path)}")
    assert_bits_equal(y.tensor, expected, what, nan_free=False)
    assert y.guards_intact(), what + ": write outside the output"
    assert x.guards_intact(), what + ": input region changed"
    return True


@pytest.mark.parametrize("align", ALIGNS)
@pytest.mark.parametrize("schedule", ["uniform", "role_split"])
@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("in_off,out_off", PATH_OFFSETS)
def test_map_parity_sizes_stages_tiles(cuda_device, op, in_off, out_off, schedule, align):
    if align == "words" and (in_off, out_off) == (0, 0):
        pytest.skip("aligned buffers: the two policies launch the same kernel")
    budget = tp.lds_budget(0)
    ran = 0
    for n in SIZES:
        x_host = workloads.uniform_pm1(n, seed=1000 + n)
        expected = oracle.pipelined_map(x_host.numpy(), op)
        for tile in TILES:
            for stages in STAGES:
                ran += _run_case(cuda_device, op, x_host, expected, in_off, out_off, tile,
                                 stages, 0, budget, schedule, align)
    assert ran > 0


@pytest.mark.parametrize("schedule", ["uniform", "role_split"])
@pytest.mark.parametrize("op", OPS)
def test_map_realign_head_and_tail(cuda_device, op, schedule):
    # heads of 0-31 floats (out 0-31 floats past a 128-byte boundary) with
    # tails of 0-3, in at several offsets, sizes around the head, one tile,
    # and one and several workgroups (the head goes to workgroup 0, the tail
    # to the last one)
    budget = tp.lds_budget(0)
    sizes = (list(range(0, 13)) + [29, 30, 31, 32, 33, 34, 35, 36, 63, 64, 65] +
             [255, 256, 257, 258, 259, 287, 288, 289, 3 * 256 + 2, 5 * 256 + 7])
    for n in sizes:
        x_host = workloads.uniform_pm1(n, seed=2000 + n)
        expected = oracle.pipelined_map(x_host.numpy(), op)
        for in_off in (0, 1, 3, 5):
            for out_off in (0, 1, 2, 3, 4, 17, 31):
                for stages, tpb in ((1, 1), (2, 1), (3, 2), (2, 0)):
                    _run_case(cuda_device, op, x_host, expected, in_off, out_off, 256, stages,
                              tpb, budget, schedule)


@pytest.mark.parametrize("schedule", ["uniform", "role_split"])
@pytest.mark.parametrize("op", OPS)
def test_map_tiles_per_block(cuda_device, op, schedule):
    budget = tp.lds_budget(0)
    n = 3 * 4096 * 5 + 13
    x_host = workloads.uniform_pm1(n, seed=77)
    expected = oracle.pipelined_map(x_host.numpy(), op)
    for tpb in (1, 2, 3, 7, 64, 1000):
        for stages in (1, 2, 4, 7):
            for tile in (256, 4096):
                _run_case(cuda_device, op, x_host, expected, 0, 0, tile, stages, tpb, budget,
                          schedule)


@pytest.mark.parametrize("align", ALIGNS)
@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("in_off,out_off", PATH_OFFSETS)
def test_map_special_values(cuda_device, op, in_off, out_off, align):
    # arbitrary bit patterns: NaN, infinities, subnormals, huge values
    g = torch.Generator().manual_seed(123)
    bits = torch.randint(-(2 ** 31), 2 ** 31, (20000,), generator=g, dtype=torch.int64)
    x_host = bits.to(torch.int32).view(torch.float32)
    specials = torch.tensor([0.0, -0.0, float("inf"), float("-inf"), 1e-45, -1e-45, 1.17e-38,
                             3.4e38, -3.4e38, 1.0, -1.0, 0.5], dtype=torch.float32)
    x_host = torch.cat([specials, x_host])
    expected = oracle.pipelined_map(x_host.numpy(), op)
    for tile, stages in ((1024, 2), (256, 1), (4096, 3)):
        _run_case(cuda_device, op, x_host, expected, in_off, out_off, tile, stages, 0,
                  tp.lds_budget(0), align=align)


@pytest.mark.parametrize("op", OPS)
def test_map_in_place(cuda_device, op):
    n = 5 * 1024 + 3
    x_host = workloads.uniform_pm1(n, seed=31)
    expected = oracle.pipelined_map(x_host.numpy(), op)
    for schedule in ("uniform", "role_split"):
        for stages in (1, 2, 4):
            for off in (0, 1, 2, 3, 8):       # in place: heads 0, 31, 30, 29, 24
                x = to_device(x_host, cuda_device, offset_words=off)
                tp.pipelined_map(x.tensor, x.tensor, op, 1024, stages, 2, schedule=schedule)
                assert_bits_equal(x.tensor, expected, f"in place {schedule} S={stages} +{off}")
                assert x.guards_intact()


def test_map_results_identical_across_parameters(cuda_device):
    # metamorphic: every (tile, stages, T, path, alignment policy) gives the same bits
    n = 100_003
    x_host = workloads.uniform_pm1(n, seed=4)
    ref = None
    budget = tp.lds_budget(0)
    for tile in (256, 1024, 8192):
        for stages in (1, 2, 3, 6):
            for tpb, schedule in ((1, "uniform"), (64, "uniform"), (3, "role_split")):
                for (in_off, out_off), align in zip(PATH_OFFSETS, ALIGNS * 3):
                    x = to_device(x_host, cuda_device, offset_words=in_off)
                    y = out_buffer(n, torch.float32, cuda_device, offset_words=out_off)
                    if tp.plan_map(x.tensor.data_ptr(), y.tensor.data_ptr(), n, "horner32", tile,
                                   stages, tpb).ring_bytes > budget:
                        continue
                    tp.pipelined_map(x.tensor, y.tensor, "horner32", tile, stages, tpb,
                                     schedule=schedule, align=align)
                    got = y.tensor.cpu()
                    if ref is None:
                        ref = got
                    assert torch.equal(got.view(torch.int32), ref.view(torch.int32))
    assert_bits_equal(ref, oracle.pipelined_map(x_host.numpy(), "horner32"), "horner32")


@pytest.mark.parametrize("op", OPS)
def test_map_residency_bound_keeps_results(cuda_device, op):
    # the LDS reserved to bound residency changes scheduling only
    n = 7 * 4096 * 3 + 5
    x_host = workloads.uniform_pm1(n, seed=55)
    expected = oracle.pipelined_map(x_host.numpy(), op)
    for tile, stages, tpb, schedule in ((256, 2, 2, "uniform"), (1024, 4, 3, "uniform"),
                                        (4096, 2, 1, "uniform"), (1024, 2, 4, "role_split")):
        for cap in (-1, 0, 1, 2, 3, 17, 40):
            for in_off, out_off in ((0, 0), (1, 0), (0, 3)):
                x = to_device(x_host, cuda_device, offset_words=in_off)
                y = out_buffer(n, torch.float32, cuda_device, offset_words=out_off)
                tp.pipelined_map(x.tensor, y.tensor, op, tile, stages, tpb, resident_cap=cap,
                                 schedule=schedule)
                what = f"{op} {schedule} tile={tile} S={stages} T={tpb} cap={cap} in_off={in_off}"
                assert_bits_equal(y.tensor, expected, what, nan_free=False)
                assert y.guards_intact() and x.guards_intact(), what


def test_map_errors(cuda_device):
    x = torch.zeros(1024, device=cuda_device)
    with pytest.raises(tp.TilepipeError) as e:
        tp.pipelined_map(x, torch.empty_like(x), "scale2", 1000, 2)
    assert e.value.status == 1
    with pytest.raises(tp.TilepipeError) as e:
        tp.pipelined_map(x[:1000], x[8:1008], "scale2", 1024, 2)
    assert e.value.status == 4
    with pytest.raises(tp.TilepipeError) as e:
        tp.pipelined_map(x, torch.empty_like(x), "scale2", 8192, 8)    # 256 KiB of LDS
    assert e.value.status == 3
    with pytest.raises(tp.TilepipeError) as e:
        tp.pipelined_map(x, torch.empty_like(x), "scale2", 1024, 2, resident_cap=-2)
    assert e.value.status == 1
    with pytest.raises(tp.TilepipeError) as e:
        tp.pipelined_map(x, torch.empty_like(x), "scale2", 1024, 2, schedule=5)
    assert e.value.status == 1
    with pytest.raises(tp.TilepipeError) as e:
        tp.pipelined_map(x, torch.empty_like(x), "scale2", 1024, 2, align=2)
    assert e.value.status == 1
