"""Maximum-size parity: problems whose byte offsets pass 2^32, so 64-bit base
arithmetic and the per-workgroup rebasing of buffer descriptors are exercised.
Inputs are generated on the device by a fixed integer pattern; sampled
windows (the start, the 4 GiB boundary, the ragged end) are brought back and
compared bit for bit with the oracle on the same input values."""
import numpy as np
import pytest
import torch

import oracle
import software_pipelining_amd as tp

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _pattern(n, dev):
    """A deterministic float32 pattern in [-0.5, 0.5): (i mod 1000003) / 1000003 - 0.5."""
    i = torch.arange(n, device=dev, dtype=torch.int64) % 1_000_003
    return i.to(torch.float32) / 1_000_003.0 - 0.5


def _check_windows(x, y, windows, op, what):
    for lo, hi in windows:
        xs = x[lo:hi].cpu().numpy()
        got = y[lo:hi].cpu().numpy()
        exp = oracle.pipelined_map(xs, op, threads=1)
        bad = np.nonzero(got.view(np.uint32) != exp.view(np.uint32))[0]
        assert bad.size == 0, f"{what} window [{lo}, {hi}): {bad.size} differ, first at {lo + bad[0]}"


@pytest.mark.parametrize("op,tile,stages,tpb", [("scale2", 256, 2, 0), ("horner32", 1024, 4, 3)])
def test_map_past_4gib(cuda_device, op, tile, stages, tpb):
    n = (1 << 30) + 7                      # 4 GiB + 28 bytes of floats, a 3-float tail
    x = _pattern(n, cuda_device)
    y = torch.full_like(x, float("nan"))
    tp.pipelined_map(x, y, op, tile, stages, tpb)
    torch.cuda.synchronize()
    edge = 1 << 30                         # element at byte 2^32
    windows = [(0, 5000), ((1 << 29) - 2000, (1 << 29) + 2000), (edge - 70_000, n)]
    _check_windows(x, y, windows, op, f"{op} n={n}")
    assert not torch.isnan(y).any().item(), "an element was not written"


def test_map_2d_past_4gib(cuda_device):
    rows, cols, ss = 65536, 16384, 16448  # a 4.3 GB source, a 4 GiB destination
    src_buf = _pattern((rows - 1) * ss + cols, cuda_device)
    src = torch.as_strided(src_buf, (rows, cols), (ss, 1))
    dst = torch.full((rows, cols), float("nan"), device=cuda_device)
    tp.map_2d(src, dst, "scale2")
    torch.cuda.synchronize()
    boundary_row = (1 << 30) // ss         # the source row that holds byte 2^32
    for r in (0, 1, boundary_row - 1, boundary_row, boundary_row + 1, rows - 2, rows - 1):
        exp = oracle.pipelined_map(src[r].cpu().numpy(), "scale2", threads=1)
        got = dst[r].cpu().numpy()
        assert np.array_equal(got.view(np.uint32), exp.view(np.uint32)), f"row {r}"
    assert not torch.isnan(dst).any().item(), "an element was not written"
