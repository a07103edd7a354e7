"""Seeded random configurations of the pipelined map (both schedules, both
alignment policies) and of the 2-D map on the GPU, each compared bit for bit
with the oracle, guard words around every buffer checked. The fixed-matrix
parity tests cover each parameter on its own; these draw them jointly (size,
offsets, tile, stages, run length, residency bound, op, box shape, strides),
so that combinations no matrix lists are exercised too ("Asynchronous Data
Movement", sections "Double buffering" and "The Tensor Memory Accelerator")."""
import numpy as np
import pytest
import torch

import oracle
import software_pipelining_amd as tp
from software_pipelining_amd import workloads
from tests.gpu_util import assert_bits_equal, out_buffer, to_device
from tests.test_gpu_map2d import _run as run_2d

pytestmark = pytest.mark.gpu

OPS = ["scale2", "horner32", "copy"]


def _map_cases(count, seed):
    rng = np.random.default_rng(seed)
    for i in range(count):
        tile = int(rng.choice([256, 512, 1024, 2048, 4096, 8192]))
        stages = int(rng.integers(1, 9))
        while stages * tile * 4 + 256 > 160 * 1024:
            stages -= 1
        n = int(rng.choice([rng.integers(0, 300), rng.integers(0, 5 * tile),
                            rng.integers(0, 40 * tile)]))
        yield dict(i=i, n=n, op=OPS[int(rng.integers(0, 3))], tile=tile, stages=stages,
                   tpb=int(rng.choice([0, 1, 2, 3, 5, 16])),
                   cap=int(rng.choice([0, 0, -1, 1, 3, 9, 20])),
                   schedule="role_split" if rng.random() < 0.25 else "uniform",
                   align="words" if rng.random() < 0.3 else "realign",
                   in_off=int(rng.integers(0, 33)), out_off=int(rng.integers(0, 33)))


@pytest.mark.parametrize("seed", [11, 12])
def test_map_random_configurations(cuda_device, seed):
    for c in _map_cases(120, seed):
        x_host = workloads.uniform_pm1(c["n"], seed=c["i"] + 1000 * seed)
        expected = oracle.pipelined_map(x_host.numpy(), c["op"])
        x = to_device(x_host, cuda_device, offset_words=c["in_off"])
        y = out_buffer(c["n"], torch.float32, cuda_device, offset_words=c["out_off"])
        tp.pipelined_map(x.tensor, y.tensor, c["op"], c["tile"], c["stages"], c["tpb"],
                         resident_cap=c["cap"], schedule=c["schedule"], align=c["align"])
        what = str(c)
        assert_bits_equal(y.tensor, expected, what, nan_free=False)
        assert y.guards_intact(), what + ": write outside the output"
        assert x.guards_intact(), what + ": input changed"


def test_map_2d_random_configurations(cuda_device):
    rng = np.random.default_rng(21)
    boxes = [(0, 0), (1, 256), (4, 256), (2, 512), (16, 64), (64, 4), (8, 1024), (1, 8192),
             (32, 32), (4, 64)]
    for i in range(100):
        rows = int(rng.choice([1, rng.integers(1, 40), rng.integers(1, 300)]))
        cols = int(rng.choice([rng.integers(1, 64), rng.integers(1, 3000)]))
        ss = cols + int(rng.integers(0, 70))
        ds = cols + int(rng.integers(0, 70))
        box = boxes[int(rng.integers(0, len(boxes)))]
        stages = int(rng.integers(1, 9))
        area = box[0] * box[1] if box[0] else 1024
        while stages * area * 4 > 160 * 1024:
            stages -= 1
        run_2d(cuda_device, OPS[int(rng.integers(0, 3))], rows, cols, ss, ds,
               int(rng.integers(0, 8)), int(rng.integers(0, 8)), box, stages,
               int(rng.choice([0, 1, 2, 3, 7])), seed=i,
               align="words" if rng.random() < 0.3 else "realign")
