"""GPU parity of tp_chunk_copy against the oracle (bit-exact), through the C ABI:
every pred/ignore_src/src_size combination, absent metadata arrays, stage
counts, tiles per workgroup, all four paths, ragged sizes, in place, and the
pre-filled destination left untouched where pred is false ("Asynchronous
Copies", section "A Global-to-Shared Copy", the paragraph on the copy's
operands)."""
import numpy as np
import pytest
import torch

import oracle
import software_pipelining_amd as tp
from software_pipelining_amd import workloads
from tests.gpu_util import Guarded, assert_bits_equal, to_device

pytestmark = pytest.mark.gpu

DEADBEEF = 0xDEADBEEF


def _dst(n_chunks, dev, off):
    return Guarded(n_chunks * 16, torch.uint8, dev, offset_words=off, fill_word=DEADBEEF)


def _meta(host, dev):
    if host is None:
        return None, None
    g = to_device(host, dev)
    return g, g.tensor


def _run(dev, inp, stages, tpb, src_off=0, dst_off=0, use=(True, True, True)):
    n = inp.src.shape[0]
    src = to_device(inp.src.reshape(-1), dev, offset_words=src_off)
    dst = _dst(n, dev, dst_off)
    metas = [m if u else None for m, u in zip((inp.pred, inp.src_size, inp.ignore_src), use)]
    devm = [_meta(m, dev) for m in metas]
    print(f"chunk_copy n={n} S={stages} T={tpb} src+{4 * src_off}B dst+{4 * dst_off}B use={use}",
          flush=True)
    path = tp.chunk_copy(src.tensor, dst.tensor, *(d[1] for d in devm), stages=stages,
                         tiles_per_block=tpb)
    expected = oracle.chunk_copy(inp.src.numpy(), inp.dst_init.numpy(),
                                 *(None if m is None else m.numpy() for m in metas))
    what = f"n={n} S={stages} T={tpb} path={int(path)} use={use}"
    if n:
        exp_path = (tp.Path.SCALAR_LOAD if src_off % 4 else 0) | (tp.Path.SCALAR_STORE if dst_off % 4 else 0)
        assert path == exp_path, what
    assert_bits_equal(dst.tensor, expected, what)
    assert dst.guards_intact(), what + ": write outside dst"
    assert src.guards_intact()
    for g, _ in devm:
        if g is not None:
            assert g.guards_intact()


def test_all_operand_combinations(cuda_device):
    pred_vals = [0, 1, 7, 255]
    ign_vals = [0, 1, 200]
    size_vals = list(range(17)) + [17, 100, 255]
    combos = [(p, g, s) for p in pred_vals for g in ign_vals for s in size_vals]
    n = len(combos)
    g = torch.Generator().manual_seed(3)
    src = torch.randint(1, 256, (n, 16), generator=g, dtype=torch.int64).to(torch.uint8)
    inp = workloads.ChunkCopyInputs(
        src=src,
        dst_init=workloads.prefill_words(n * 4).view(torch.uint8).reshape(n, 16),
        pred=torch.tensor([c[0] for c in combos], dtype=torch.uint8),
        src_size=torch.tensor([c[2] for c in combos], dtype=torch.uint8),
        ignore_src=torch.tensor([c[1] for c in combos], dtype=torch.uint8))
    for stages in (1, 2, 3):
        for src_off, dst_off in ((0, 0), (1, 0), (0, 1), (2, 3)):
            _run(cuda_device, inp, stages, 0, src_off, dst_off)


SIZES = [0, 1, 3, 255, 256, 257, 1000, 64 * 256 + 1, 3 * 64 * 256 + 100]


@pytest.mark.parametrize("src_off,dst_off", [(0, 0), (1, 0), (0, 1), (3, 2)])
def test_chunk_copy_sizes_and_stages(cuda_device, src_off, dst_off):
    budget = tp.lds_budget(0)
    for n in SIZES:
        inp = workloads.chunk_copy_inputs(n, seed=50 + n)
        for stages in (1, 2, 3, 4, 6, 8):
            if tp.plan_chunk_copy(16, 16 * (n + 1) + 64, n, stages=stages).lds_bytes > budget:
                continue
            _run(cuda_device, inp, stages, 0, src_off, dst_off)


def test_chunk_copy_tiles_per_block(cuda_device):
    inp = workloads.chunk_copy_inputs(10 * 256 + 17, seed=9)
    for tpb in (1, 2, 3, 5, 64):
        for stages in (1, 2, 5):
            _run(cuda_device, inp, stages, tpb)


@pytest.mark.parametrize("use", [(False, False, False), (True, False, False), (False, True, False),
                                 (False, False, True), (True, True, False), (False, True, True)])
def test_absent_metadata_defaults(cuda_device, use):
    inp = workloads.chunk_copy_inputs(5000, seed=11, p_pred=0.5, p_ignore=0.2)
    for stages in (1, 2, 4):
        _run(cuda_device, inp, stages, 0, use=use)


def test_all_pred_false_leaves_destination(cuda_device):
    n = 4096 + 5
    inp = workloads.chunk_copy_inputs(n, seed=2)
    inp.pred.zero_()
    _run(cuda_device, inp, 2, 0)


def test_chunk_copy_in_place(cuda_device):
    n = 3000
    inp = workloads.chunk_copy_inputs(n, seed=21)
    expected = oracle.chunk_copy(inp.src.numpy(), inp.src.numpy(), inp.pred.numpy(),
                                 inp.src_size.numpy(), inp.ignore_src.numpy())
    for stages in (1, 2, 3):
        buf = to_device(inp.src.reshape(-1), cuda_device)
        metas = [to_device(m, cuda_device) for m in (inp.pred, inp.src_size, inp.ignore_src)]
        print(f"chunk_copy in place n={n} S={stages}", flush=True)
        tp.chunk_copy(buf.tensor, buf.tensor, *(m.tensor for m in metas), stages=stages)
        assert_bits_equal(buf.tensor, expected, f"in place S={stages}")
        assert buf.guards_intact()


def test_chunk_copy_errors(cuda_device):
    src = torch.zeros(64 * 16, dtype=torch.uint8, device=cuda_device)
    dst = torch.zeros(64 * 16 + 64, dtype=torch.uint8, device=cuda_device)
    with pytest.raises(tp.TilepipeError) as e:      # dst overlaps the pred array
        tp.chunk_copy(src, dst[:64 * 16], pred=dst[64 * 16 - 32:64 * 16 + 32])
    assert e.value.status == 4
    with pytest.raises(tp.TilepipeError) as e:      # src not 4-byte aligned
        tp.chunk_copy(dst[1:64 * 16 + 1], src)
    assert e.value.status == 2
    with pytest.raises(tp.TilepipeError) as e:
        tp.chunk_copy(src, dst[:64 * 16], stages=0)
    assert e.value.status == 1


@pytest.mark.parametrize("width", [4, 8])
def test_narrow_chunks(cuda_device, width):
    # 4- and 8-byte chunks: every operand combination, absent arrays, stages, runs
    rng = np.random.default_rng(width)
    for n in (1, 255, 256, 1000, 5 * 256 + 77):
        src_h = rng.integers(0, 256, size=n * width, dtype=np.uint8)
        dst_h = np.frombuffer(np.full(-(-n * width // 4), DEADBEEF, np.uint32).tobytes(),
                              np.uint8)[:n * width].copy()
        pred_h = rng.integers(0, 3, size=n).astype(np.uint8)          # 0 false, 1-2 true
        size_h = rng.integers(0, width + 3, size=n).astype(np.uint8)  # past width: clamped
        ign_h = (rng.random(n) < 0.05).astype(np.uint8)
        for stages in (1, 2, 4):
            for tpb in (0, 1, 3):
                for use in ((True, True, True), (False, True, False), (False, False, False)):
                    metas = [m if u else None for m, u in zip((pred_h, size_h, ign_h), use)]
                    src = to_device(torch.from_numpy(src_h), cuda_device)
                    dst = Guarded(n * width, torch.uint8, cuda_device, fill_word=DEADBEEF)
                    devm = [_meta(None if m is None else torch.from_numpy(m), cuda_device)
                            for m in metas]
                    print(f"chunk_copy W={width} n={n} S={stages} T={tpb} use={use}", flush=True)
                    path = tp.chunk_copy(src.tensor, dst.tensor, *(d[1] for d in devm),
                                         stages=stages, tiles_per_block=tpb, chunk_bytes=width)
                    assert path == tp.Path.SCALAR
                    expected = oracle.chunk_copy(src_h, dst_h, *metas, chunk_bytes=width)
                    what = f"W={width} n={n} S={stages} T={tpb} use={use}"
                    assert_bits_equal(dst.tensor, expected, what)
                    assert dst.guards_intact() and src.guards_intact(), what
