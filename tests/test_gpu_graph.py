"""The entry points inside a captured HIP graph: they allocate nothing, set
nothing with memset and never synchronize, so a graph that records them can be
replayed. Each replay is checked against the oracle, with eager work and
synchronizations between the replays, and the inputs changed in place between
replays so a replay that reused stale results would be caught."""
import numpy as np
import pytest
import torch

import oracle
import software_pipelining_amd as tp
from software_pipelining_amd import workloads

pytestmark = pytest.mark.gpu


def test_graph_replays_match_the_oracle(cuda_device):
    dev = cuda_device
    a = workloads.arange_rows(64).to(dev)
    b = torch.empty_like(a)
    x = workloads.uniform_pm1(3 * 1024 + 5, seed=11).to(dev)
    y = torch.empty_like(x)
    s2 = workloads.uniform_pm1(40 * 300, seed=12).to(dev).view(40, 300)
    d2 = torch.zeros(40, 260, device=dev)
    src2 = s2[:, :260]

    def work():
        tp.row_shift(a, b)
        tp.pipelined_map(x, y, "horner32", 1024, 2, 2)
        tp.map_2d(src2, d2, "scale2")

    work()                                   # first calls outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for rep in range(4):
        # new inputs in place, eager work of the program's own, then a replay
        a.copy_(workloads.random_rows(64, seed=100 + rep).to(dev))
        x.copy_(workloads.uniform_pm1(x.numel(), seed=200 + rep).to(dev))
        s2.copy_(workloads.uniform_pm1(s2.numel(), seed=300 + rep).to(dev).view(40, 300))
        junk = torch.randn(1 << 16, device=dev).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(b.cpu().numpy().view(np.uint32),
                              oracle.row_shift(a.cpu().numpy()).view(np.uint32)), rep
        assert np.array_equal(y.cpu().numpy().view(np.uint32),
                              oracle.pipelined_map(x.cpu().numpy(), "horner32").view(np.uint32)), rep
        exp2 = np.zeros((40, 260), np.float32)
        oracle.map_2d(s2.cpu().numpy()[:, :260], exp2, "scale2")
        assert np.array_equal(d2.cpu().numpy().view(np.uint32), exp2.view(np.uint32)), rep
        del junk
