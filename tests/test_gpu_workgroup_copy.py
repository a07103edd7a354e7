"""GPU parity of tp_workgroup_copy against the oracle (bit-exact), through the
C ABI: chunk k of the source, loaded into workgroup k's LDS, is handed to
workgroup k + 1 through a staging slot of tagged 8-byte words and written as
chunk k + 1 of the destination ("Asynchronous Copies", section "Copies between
CTAs"). Guard words around every buffer catch a write outside it. A tiny spin
limit, set from the host, makes receivers give up early: every chunk must then
be either the received one or untouched, and the status must say so."""
import numpy as np
import pytest
import torch

import oracle
import software_pipelining_amd as tp
from tests.gpu_util import Guarded, assert_bits_equal, to_device

pytestmark = pytest.mark.gpu

CHUNK = 256
DEADBEEF = 0xDEADBEEF


def _case(dev, n, seed, src_off=0, dst_off=0):
    rng = np.random.default_rng(seed)
    src_h = rng.integers(0, 256, n * CHUNK, dtype=np.uint8)
    src = to_device(torch.from_numpy(src_h), dev, offset_words=src_off)
    dst = Guarded(n * CHUNK, torch.uint8, dev, offset_words=dst_off, fill_word=DEADBEEF)
    dst_h = dst.tensor.cpu().numpy().copy()
    ws = Guarded(max(4, tp.workgroup_copy_workspace_bytes(n)), torch.uint8, dev, fill_word=0xFFFFFFFF)
    status = Guarded(4, torch.int32, dev, fill_word=7)
    return src_h, src, dst_h, dst, ws, status


@pytest.mark.parametrize("n", [1, 2, 3, 64, 257, 1000, 5000, 1 << 16])
def test_matches_oracle(cuda_device, n):
    for src_off, dst_off in ((0, 0), (1, 3)):
        src_h, src, dst_h, dst, ws, status = _case(cuda_device, n, n, src_off, dst_off)
        print(f"workgroup_copy n={n} src+{4 * src_off}B dst+{4 * dst_off}B", flush=True)
        tp.workgroup_copy(src.tensor, dst.tensor, ws.tensor, status.tensor)
        assert_bits_equal(dst.tensor, oracle.workgroup_copy(src_h, dst_h), f"n={n}")
        assert int(status.tensor.item()) == 0
        for g in (src, dst, ws, status):
            assert g.guards_intact(), f"n={n}: write outside a buffer"


def test_repeated_calls_new_data(cuda_device):
    # ten calls in a row on one workspace, each with new data over 2^18
    # chunks: a receiver that read its slot before the sender's bytes were
    # visible would return the previous call's bytes
    n = 1 << 18
    ws = torch.empty(tp.workgroup_copy_workspace_bytes(n), dtype=torch.uint8, device=cuda_device)
    status = torch.empty(1, dtype=torch.int32, device=cuda_device)
    dst = torch.empty(n * CHUNK, dtype=torch.uint8, device=cuda_device)
    for it in range(10):
        g = torch.Generator().manual_seed(1000 + it)
        src = torch.randint(0, 256, (n * CHUNK,), generator=g, dtype=torch.uint8).to(cuda_device)
        dst.fill_(it)
        print(f"workgroup_copy n={n} call {it}", flush=True)
        tp.workgroup_copy(src, dst, ws, status)
        assert int(status.item()) == 0
        assert torch.equal(dst[CHUNK:], src[:-CHUNK]), f"call {it}"
        assert bool((dst[:CHUNK] == it).all())


def test_large(cuda_device):
    n = 1 << 20                                   # 256 MiB each way
    g = torch.Generator().manual_seed(8)
    src_h = torch.randint(0, 256, (n * CHUNK,), generator=g, dtype=torch.uint8)
    src = src_h.to(cuda_device)
    dst = torch.zeros(n * CHUNK, dtype=torch.uint8, device=cuda_device)
    print(f"workgroup_copy n={n}", flush=True)
    status = tp.workgroup_copy(src, dst)
    assert int(status.item()) == 0
    assert torch.equal(dst[CHUNK:], src[:-CHUNK]) and int(dst[:CHUNK].sum().item()) == 0


def test_in_place_and_workspace_reuse(cuda_device):
    n = 3000
    ws = torch.empty(tp.workgroup_copy_workspace_bytes(n), dtype=torch.uint8, device=cuda_device)
    status = torch.empty(1, dtype=torch.int32, device=cuda_device)
    rng = np.random.default_rng(4)
    for it in range(3):                            # the same workspace, three calls in a row
        h = rng.integers(0, 256, n * CHUNK, dtype=np.uint8)
        buf = torch.from_numpy(h).to(cuda_device)
        print(f"workgroup_copy in place n={n} call {it}", flush=True)
        tp.workgroup_copy(buf, buf, ws, status)
        assert_bits_equal(buf, oracle.workgroup_copy(h, h), f"in place call {it}")
        assert int(status.item()) == 0


def test_graph_replays(cuda_device):
    # the clearing kernel and the hand-off kernel captured once and replayed,
    # with the source changed and eager work between replays
    n = 2048
    src = torch.zeros(n * CHUNK, dtype=torch.uint8, device=cuda_device)
    dst = torch.zeros_like(src)
    ws = torch.empty(tp.workgroup_copy_workspace_bytes(n), dtype=torch.uint8, device=cuda_device)
    status = torch.empty(1, dtype=torch.int32, device=cuda_device)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        tp.workgroup_copy(src, dst, ws, status)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        tp.workgroup_copy(src, dst, ws, status)
    rng = np.random.default_rng(6)
    for r in range(4):
        h = rng.integers(0, 256, n * CHUNK, dtype=np.uint8)
        src.copy_(torch.from_numpy(h))
        dst.fill_(r)
        torch.cuda.synchronize()
        print(f"workgroup_copy graph replay {r}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        exp = oracle.workgroup_copy(h, np.full(n * CHUNK, r, np.uint8))
        assert_bits_equal(dst, exp, f"replay {r}")
        assert int(status.item()) == 0


def test_tiny_spin_limit_gives_up_cleanly(cuda_device):
    # one poll per receiver: some receivers may find their slot not yet
    # tagged and give up;
    # every chunk is then either the received one or untouched, and the status
    # is 1 exactly when some chunk was not written
    n = 1 << 14
    for seed in range(3):
        src_h, src, dst_h, dst, ws, status = _case(cuda_device, n, 100 + seed)
        print(f"workgroup_copy n={n} spin_limit=1 seed={seed}", flush=True)
        tp.workgroup_copy(src.tensor, dst.tensor, ws.tensor, status.tensor, spin_limit=1)
        got = dst.tensor.cpu().numpy().reshape(n, CHUNK)
        exp = oracle.workgroup_copy(src_h, dst_h).reshape(n, CHUNK)
        untouched = dst_h.reshape(n, CHUNK)
        ok = np.all(got == exp, axis=1)
        kept = np.all(got == untouched, axis=1)
        assert np.all(ok | kept), "a chunk is neither received nor untouched"
        st = int(status.tensor.item())
        missing = int(np.sum(~ok[1:]))
        assert st in (0, 1) and (st == 1) == (missing > 0), (st, missing)
        assert dst.guards_intact() and ws.guards_intact()


def test_errors(cuda_device):
    n = 16
    src = torch.zeros(n * CHUNK, dtype=torch.uint8, device=cuda_device)
    dst = torch.zeros_like(src)
    status = torch.empty(1, dtype=torch.int32, device=cuda_device)
    short = torch.empty(tp.workgroup_copy_workspace_bytes(n) - 1, dtype=torch.uint8,
                        device=cuda_device)
    with pytest.raises(tp.TilepipeError) as e:
        tp.workgroup_copy(src, dst, short, status)
    assert e.value.status == 1
    big = torch.zeros(4 * n * CHUNK, dtype=torch.uint8, device=cuda_device)
    with pytest.raises(tp.TilepipeError) as e:       # dst overlapping src in part
        tp.workgroup_copy(big[:n * CHUNK], big[CHUNK:(n + 1) * CHUNK])
    assert e.value.status == 4
    need = tp.workgroup_copy_workspace_bytes(n)
    with pytest.raises(tp.TilepipeError) as e:       # the workspace over dst's last chunk
        tp.workgroup_copy(src, big[:n * CHUNK], big[(n - 1) * CHUNK:(n - 1) * CHUNK + need], status)
    assert e.value.status == 4
    with pytest.raises(tp.TilepipeError) as e:
        tp.workgroup_copy(src, dst, spin_limit=-1)
    assert e.value.status == 1
