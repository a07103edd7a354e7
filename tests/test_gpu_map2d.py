"""GPU parity of tp_map_2d against the oracle (bit-exact), through the C ABI:
windows of row-major matrices with row strides, every op, ragged edges that
cut boxes, several box shapes, stages and runs, both alignment policies (all
four load/store paths) and in-place use. The whole destination buffer is compared, so elements between
the rows and around the window must come back untouched ("Asynchronous Data
Movement", section "The Tensor Memory Accelerator": a tile described by a
base, a shape and strides)."""
import numpy as np
import pytest
import torch

import oracle
import software_pipelining_amd as tp
from software_pipelining_amd import workloads

pytestmark = pytest.mark.gpu

SENTINEL = np.float32(-7.25)
GUARD = 64


def _buffers(rows, cols, stride, off, seed):
    """A host buffer holding a (rows, cols) window at float offset GUARD + off
    with the given row stride, filled with seeded values."""
    n = GUARD + off + (rows - 1) * stride + cols + GUARD if rows and cols else 2 * GUARD
    return workloads.uniform_pm1(n, seed=seed).numpy()


def _view_np(buf, rows, cols, stride, off):
    return np.lib.stride_tricks.as_strided(buf[GUARD + off:], shape=(rows, cols),
                                           strides=(stride * 4, 4))


def _view_t(buf, rows, cols, stride, off):
    return torch.as_strided(buf, (rows, cols), (stride, 1), GUARD + off)


def _run(dev, op, rows, cols, ss, ds, soff, doff, box, stages, tpb, seed=0, align="realign"):
    src_h = _buffers(rows, cols, ss, soff, seed=100 + seed)
    dst_h = np.full(_buffers(rows, cols, ds, doff, seed=1).size, SENTINEL, np.float32)
    expect = dst_h.copy()
    if rows and cols:
        oracle.map_2d(_view_np(src_h, rows, cols, ss, soff), _view_np(expect, rows, cols, ds, doff), op)
    src = torch.from_numpy(src_h).to(dev)
    dst = torch.from_numpy(dst_h).to(dev)
    path = tp.map_2d(_view_t(src, rows, cols, ss, soff), _view_t(dst, rows, cols, ds, doff), op,
                     box[0], box[1], stages, tpb, align=align)
    got = dst.cpu().numpy()
    what = (f"{op} {align} {rows}x{cols} ss={ss} ds={ds} off={soff},{doff} box={box} S={stages} "
            f"T={tpb} path={int(path)}")
    bad = np.nonzero(got.view(np.uint32) != expect.view(np.uint32))[0]
    assert bad.size == 0, f"{what}: {bad.size} differ, first at {bad[:6].tolist()}"
    assert torch.equal(src.cpu(), torch.from_numpy(src_h)), what + ": source changed"
    return path


SHAPES = [(1, 1), (1, 300), (3, 5), (5, 4), (17, 300), (64, 256), (100, 1000), (257, 64),
          (33, 8200)]
BOXES = [(1, 256), (4, 256), (2, 512), (16, 64), (64, 4), (1, 8192), (8, 1024), (0, 0)]


@pytest.mark.parametrize("align", ["realign", "words"])
@pytest.mark.parametrize("op", ["scale2", "horner32", "copy"])
def test_map_2d_parity_shapes_boxes(cuda_device, op, align):
    for i, (rows, cols) in enumerate(SHAPES):
        for box in BOXES:
            for ss, ds in ((cols, cols), (cols + 4, cols + 12), (cols + 3, cols + 1)):
                path = _run(cuda_device, op, rows, cols, ss, ds, 0, 0, box, 2, 0, seed=i,
                            align=align)
                if align == "realign":
                    assert path == (tp.Path.X4 if cols % 4 == 0 else tp.Path.SCALAR)


@pytest.mark.parametrize("op", ["scale2", "copy"])
def test_map_2d_stages_runs_paths(cuda_device, op):
    rows, cols = 70, 1028
    for soff, doff, want in ((0, 0, tp.Path.X4), (1, 0, tp.Path.SCALAR_LOAD),
                             (0, 2, tp.Path.SCALAR_STORE), (3, 1, tp.Path.SCALAR)):
        for stages in (1, 2, 3, 4, 8):
            for tpb in (1, 2, 3, 64):
                for align in ("realign", "words"):
                    path = _run(cuda_device, op, rows, cols, cols + 4, cols + 8, soff, doff,
                                (4, 256), stages, tpb, align=align)
                    assert path == (want if align == "words" else tp.Path.X4)


def test_map_2d_in_place_and_empty(cuda_device):
    rows, cols, stride = 45, 515, 520
    host = _buffers(rows, cols, stride, 0, seed=5)
    expect = host.copy()
    oracle.map_2d(_view_np(host, rows, cols, stride, 0), _view_np(expect, rows, cols, stride, 0),
                  "horner32")
    buf = torch.from_numpy(host).to(cuda_device)
    v = _view_t(buf, rows, cols, stride, 0)
    tp.map_2d(v, v, "horner32", 2, 512, 2, 2)
    assert np.array_equal(buf.cpu().numpy().view(np.uint32), expect.view(np.uint32))
    # nothing to do: no launch, nothing written
    before = buf.clone()
    tp.map_2d(v[:0], v[:0], "scale2")
    tp.map_2d(v[:, :0], v[:, :0], "scale2")
    assert torch.equal(buf, before)


def test_map_2d_errors(cuda_device):
    buf = torch.zeros(100_000, device=cuda_device)
    a = torch.as_strided(buf, (10, 100), (100, 1), 0)
    b = torch.as_strided(buf, (10, 100), (100, 1), 500)       # overlaps a's range
    with pytest.raises(tp.TilepipeError) as e:
        tp.map_2d(a, b, "scale2")
    assert e.value.status == 4
    c = torch.as_strided(buf, (10, 100), (100, 1), 50_000)
    with pytest.raises(tp.TilepipeError) as e:
        tp.map_2d(a, c, "scale2", 3, 256)                       # box_rows not a power of two
    assert e.value.status == 1
    with pytest.raises(tp.TilepipeError) as e:
        tp.map_2d(a, c, "scale2", align=3)
    assert e.value.status == 1
