"""The allocation-free copy between workgroups (tp_workgroup_copy_noalloc,
through the C ABI) against the entry point that takes a caller workspace
(tp_workgroup_copy): bit-exact on two calls in a row, the second smaller, so
the static workspace keeps the first call's tagged slots when the second
runs. Both are also checked against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import software_pipelining_amd as tp

pytestmark = pytest.mark.gpu

CHUNK = 256


def test_noalloc_matches_workspace_entry_point(cuda_device):
    rng = np.random.default_rng(12)
    status_a = torch.empty(1, dtype=torch.int32, device=cuda_device)
    status_b = torch.empty(1, dtype=torch.int32, device=cuda_device)
    for n in (16384, 3001):                        # the maximum, then a smaller call
        src_h = rng.integers(0, 256, n * CHUNK, dtype=np.uint8)
        init = rng.integers(0, 256, n * CHUNK, dtype=np.uint8)
        src = torch.from_numpy(src_h).to(cuda_device)
        dst_a = torch.from_numpy(init).to(cuda_device)
        dst_b = torch.from_numpy(init).to(cuda_device)
        ws = torch.empty(tp.workgroup_copy_workspace_bytes(n), dtype=torch.uint8,
                         device=cuda_device)
        print(f"workgroup_copy_noalloc n={n}", flush=True)
        tp.workgroup_copy_noalloc(src, dst_a, status_a)
        tp.workgroup_copy(src, dst_b, ws, status_b)
        torch.cuda.synchronize()
        assert int(status_a.item()) == 0 and int(status_b.item()) == 0
        assert torch.equal(dst_a, dst_b), f"n={n}: the two entry points differ"
        assert np.array_equal(dst_a.cpu().numpy(), oracle.workgroup_copy(src_h, init)), f"n={n}"


def test_noalloc_rejects_more_than_its_workspace_holds(cuda_device):
    n = 16385
    src = torch.zeros(n * CHUNK, dtype=torch.uint8, device=cuda_device)
    status = torch.empty(1, dtype=torch.int32, device=cuda_device)
    with pytest.raises(tp.TilepipeError) as e:
        tp.workgroup_copy_noalloc(src, torch.zeros_like(src), status)
    assert e.value.status == 1
