"""GPU parity of tp_row_shift against the oracle (bit-exact), through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import software_pipelining_amd as tp
from software_pipelining_amd import workloads
from tests.gpu_util import assert_bits_equal, out_buffer, to_device

pytestmark = pytest.mark.gpu


def test_device_is_gfx950(cuda_device):
    tp.device_check(0)
    assert tp.lds_budget(0) >= 64 * 1024


def test_worked_example_64x4(cuda_device):
    # "Asynchronous Copies", "A Global-to-Shared Copy": arange(256) as 64x4,
    # one 64-lane workgroup, B = roll(A, -1, dims=0)
    a_host = workloads.arange_rows(64)
    a = to_device(a_host, cuda_device)
    b = out_buffer(256, torch.float32, cuda_device)
    path = tp.row_shift(a.tensor.view(64, 4), b.tensor.view(64, 4))
    assert path == tp.Path.X4
    expected = oracle.row_shift(a_host.numpy())
    assert_bits_equal(b.tensor, expected, "row shift 64x4")
    assert torch.equal(b.tensor.view(64, 4).cpu(), torch.roll(a_host, -1, 0))
    assert b.guards_intact()


@pytest.mark.parametrize("rows", [1, 2, 3, 63, 64, 65, 127, 128, 500, 1023, 1024])
@pytest.mark.parametrize("a_off,b_off", [(0, 0), (1, 0), (0, 3), (2, 1)])
def test_row_shift_bitwise(cuda_device, rows, a_off, b_off):
    a_host = workloads.random_rows(rows, seed=rows * 7 + a_off)   # arbitrary bits, NaNs too
    a = to_device(a_host, cuda_device, offset_words=a_off)
    b = out_buffer(rows * 4, torch.float32, cuda_device, offset_words=b_off)
    path = tp.row_shift(a.tensor.view(rows, 4), b.tensor.view(rows, 4))
    expect_path = (tp.Path.SCALAR_LOAD if a_off % 4 else 0) | (tp.Path.SCALAR_STORE if b_off % 4 else 0)
    assert path == expect_path
    assert_bits_equal(b.tensor, oracle.row_shift(a_host.numpy()), f"rows={rows} path={path}")
    assert a.guards_intact() and b.guards_intact()


@pytest.mark.parametrize("rows", [1, 64, 333, 1024])
def test_row_shift_in_place(cuda_device, rows):
    a_host = workloads.random_rows(rows, seed=900 + rows)
    a = to_device(a_host, cuda_device)
    t = a.tensor.view(rows, 4)
    tp.row_shift(t, t)
    assert_bits_equal(a.tensor, oracle.row_shift(a_host.numpy()), "in place")
    assert a.guards_intact()


def test_row_shift_repeated_is_identity(cuda_device):
    rows = 96
    a_host = workloads.random_rows(rows, seed=5)
    a = to_device(a_host, cuda_device)
    t = a.tensor.view(rows, 4)
    for _ in range(rows):
        tp.row_shift(t, t)
    assert_bits_equal(a.tensor, a_host.numpy(), "rows shifts")


def test_row_shift_errors(cuda_device):
    a = torch.zeros(1025, 4, device=cuda_device)
    with pytest.raises(tp.TilepipeError) as e:
        tp.row_shift(a, torch.empty_like(a))
    assert e.value.status == 1
    z = torch.zeros(0, 4, device=cuda_device)
    assert tp.row_shift(z, torch.empty_like(z)) == tp.Path.X4
    buf = torch.zeros(130 * 4, device=cuda_device)
    with pytest.raises(tp.TilepipeError) as e:                 # partial overlap
        tp.row_shift(buf[:128 * 4].view(128, 4), buf[4:129 * 4].view(128, 4))
    assert e.value.status == 4
