"""Helpers for the GPU parity tests: offset allocations with guard regions and
bitwise comparison against oracle outputs."""
from __future__ import annotations

import numpy as np
import torch

GUARD = 64                      # sentinel words before and after every buffer
SENTINEL = 0x7FC0DEAD           # a NaN pattern none of the tests' results contain


def _i32(u: int) -> int:
    return u - (1 << 32) if u >= (1 << 31) else u


class Guarded:
    """`nbytes` of device memory at a word offset inside a larger allocation
    (so its alignment is chosen by the test), with sentinel words around it
    that any stray write would change."""

    def __init__(self, nbytes: int, dtype: torch.dtype, device, offset_words: int = 0,
                 fill_word: int | None = None):
        words = (nbytes + 3) // 4
        self.lo = GUARD + offset_words
        self.hi = self.lo + words
        self.raw = torch.full((self.hi + GUARD,), _i32(SENTINEL), dtype=torch.int32, device=device)
        if fill_word is not None:
            self.raw[self.lo:self.hi] = _i32(fill_word)
        self.tensor = self.raw[self.lo:self.hi].view(torch.uint8)[:nbytes].view(dtype)

    def guards_intact(self) -> bool:
        s = _i32(SENTINEL)
        return bool((self.raw[:self.lo] == s).all().item()) and bool((self.raw[self.hi:] == s).all().item())


def to_device(host: torch.Tensor, device, offset_words: int = 0) -> Guarded:
    g = Guarded(host.numel() * host.element_size(), host.dtype, device, offset_words)
    if host.numel():
        g.tensor.copy_(host.reshape(-1))
    return g


def out_buffer(n: int, dtype: torch.dtype, device, offset_words: int = 0,
               fill_word: int = 0xFFFFFFFF) -> Guarded:
    esize = torch.empty(0, dtype=dtype).element_size()
    return Guarded(n * esize, dtype, device, offset_words, fill_word)


def assert_bits_equal(got: torch.Tensor, expected: np.ndarray, what: str, nan_free: bool = True):
    """Bitwise equality of a GPU float32/uint8 tensor with a numpy array.
    With nan_free False, positions where `expected` is NaN only need a NaN
    (the payload of a NaN result is not fixed)."""
    g = got.detach().reshape(-1).cpu().numpy()
    e = np.ascontiguousarray(expected).reshape(-1)
    assert g.shape == e.shape, (what, g.shape, e.shape)
    if g.dtype == np.float32:
        gb, eb = g.view(np.uint32), e.view(np.uint32)
        if not nan_free:
            en = np.isnan(e)
            assert np.all(np.isnan(g[en])), f"{what}: NaN expected but not produced"
            gb, eb = gb[~en], eb[~en]
    else:
        gb, eb = g, e
    bad = np.nonzero(gb != eb)[0]
    if bad.size:
        i = bad[:8]
        raise AssertionError(f"{what}: {bad.size} of {eb.size} differ, first at {i.tolist()}: "
                             f"got {[hex(int(v)) for v in gb[i]]} expected {[hex(int(v)) for v in eb[i]]}")


def assert_equal_on_device(got: torch.Tensor, expected: torch.Tensor, what: str):
    """Bitwise equality of two same-size tensors, compared on the GPU (for
    full-size workloads); reports the first differing positions."""
    a = got.reshape(-1).view(torch.uint8) if got.dtype == torch.uint8 else got.reshape(-1).view(torch.int32)
    b = expected.reshape(-1).view(torch.uint8) if expected.dtype == torch.uint8 else expected.reshape(-1).view(torch.int32)
    assert a.numel() == b.numel(), (what, a.numel(), b.numel())
    ne = a != b
    n_bad = int(ne.sum().item())
    if n_bad:
        idx = torch.nonzero(ne)[:8].reshape(-1)
        raise AssertionError(f"{what}: {n_bad} of {a.numel()} differ, first at {idx.tolist()}: "
                             f"got {a[idx].tolist()} expected {b[idx].tolist()}")
