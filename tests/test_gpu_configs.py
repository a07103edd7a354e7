"""The five workloads at full size, bit-exact against the oracle on the same
host inputs, in the launch configurations the benchmark times.

1. row exchange of the 64x4 worked example;
2. double-buffered scale-by-2, 2^24 floats, tile 256, 2 stages, 64 tiles/WG;
3. stage/tile sweep of scale-by-2 over 2^28 floats, stages 1-4 x tiles
   256/1024/4096, aligned and with a 4-byte source offset (16-byte loads at that
   offset, and the pages' 4-byte fallback);
4. predicated chunk copy of 2^26 chunks;
5. 32-step fmaf Horner chain over 2^27 floats, tile 1024, stages 1/2/4.
"""
import numpy as np
import pytest
import torch

import oracle
import software_pipelining_amd as tp
from software_pipelining_amd import workloads
from tests.gpu_util import assert_equal_on_device

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def test_config1_row_shift(cuda_device):
    a = workloads.arange_rows(64)
    b = torch.full((64, 4), float("nan"), device=cuda_device)
    assert tp.row_shift(a.to(cuda_device), b) == tp.Path.X4
    exp = torch.from_numpy(oracle.row_shift(a.numpy())).to(cuda_device)
    assert_equal_on_device(b, exp, "config 1")


def test_config2_double_buffered_scale2(cuda_device):
    n = 1 << 24
    x_host = workloads.uniform_pm1(n, seed=1)
    exp = torch.from_numpy(oracle.pipelined_map(x_host.numpy(), "scale2")).to(cuda_device)
    x = x_host.to(cuda_device)
    y = torch.full_like(x, float("nan"))
    assert tp.pipelined_map(x, y, "scale2", 256, 2, 64) == tp.Path.X4
    assert_equal_on_device(y, exp, "config 2")


def test_config3_stage_tile_sweep(cuda_device):
    n = 1 << 28
    x_host = workloads.uniform_pm1(n, seed=2)
    xbuf = torch.empty(n + 4, dtype=torch.float32, device=cuda_device)
    xbuf[:n].copy_(x_host)
    xbuf[n:] = 0.5
    y = torch.empty(n, dtype=torch.float32, device=cuda_device)
    for off in (0, 1):
        host_in = x_host.numpy() if off == 0 else np.concatenate([x_host.numpy()[1:], [np.float32(0.5)]])
        exp = torch.from_numpy(oracle.pipelined_map(host_in, "scale2")).to(cuda_device)
        xin = xbuf[off:off + n]
        for tile in (256, 1024, 4096):
            for stages in (1, 2, 3, 4):
                # the library's run length (as benchmarked) and 64, and with the
                # offset source both alignment policies
                for tpb, align in ((0, "realign"), (64, "realign"), (0, "words")):
                    if align == "words" and not off:
                        continue
                    y.fill_(float("nan"))
                    path = tp.pipelined_map(xin, y, "scale2", tile, stages, tpb, align=align)
                    assert path == (tp.Path.SCALAR_LOAD if align == "words" else tp.Path.X4)
                    assert_equal_on_device(y, exp, f"config 3 offset={4 * off}B tile={tile} "
                                                   f"S={stages} T={tpb} {align}")
        del exp


def test_config4_predicated_chunk_copy(cuda_device):
    nc = 1 << 26
    inp = workloads.chunk_copy_inputs(nc, seed=3)
    exp = oracle.chunk_copy(inp.src.numpy(), inp.dst_init.numpy(), inp.pred.numpy(),
                            inp.src_size.numpy(), inp.ignore_src.numpy())
    exp_d = torch.from_numpy(exp.reshape(-1)).to(cuda_device)
    src = inp.src.reshape(-1).to(cuda_device)
    meta = [m.to(cuda_device) for m in (inp.pred, inp.src_size, inp.ignore_src)]
    # the launches the benchmark times: the default runs (max(1, S-1) tiles) at
    # 1-4 stages, and runs of 2, 8 and 64 tiles at 2 stages
    for stages, tpb in ((1, 0), (2, 0), (3, 0), (4, 0), (2, 2), (2, 8), (2, 64)):
        dst = inp.dst_init.reshape(-1).to(cuda_device)
        print(f"config 4 chunk_copy n=2^26 S={stages} T={tpb}", flush=True)
        tp.chunk_copy(src, dst, *meta, stages=stages, tiles_per_block=tpb)
        assert_equal_on_device(dst, exp_d, f"config 4 S={stages} T={tpb}")


def test_config5_horner32(cuda_device):
    n = 1 << 27
    x_host = workloads.uniform_pm1(n, seed=4)
    exp_host = oracle.pipelined_map(x_host.numpy(), "horner32")
    assert oracle.horner32_subnormal_steps(x_host.numpy()) == 0
    exp = torch.from_numpy(exp_host).to(cuda_device)
    x = x_host.to(cuda_device)
    y = torch.empty_like(x)
    for stages in (1, 2, 4):
        for tpb, cap, schedule in ((0, 0, "uniform"), (16, 0, "uniform"), (64, 0, "uniform"),
                                   (8, 2, "uniform"), (0, 0, "role_split"), (8, 2, "role_split")):
            y.fill_(float("nan"))
            tp.pipelined_map(x, y, "horner32", 1024, stages, tpb, resident_cap=cap,
                             schedule=schedule)
            assert_equal_on_device(y, exp, f"config 5 {schedule} S={stages} T={tpb} cap={cap}")
