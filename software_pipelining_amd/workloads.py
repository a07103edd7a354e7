"""Seeded synthetic inputs for libtilepipe's workloads.

This module only draws inputs; it holds none of the operations' arithmetic, so
the GPU path and the CPU oracle can both be fed from it without sharing any
computation. Every array comes from torch's CPU generator with a fixed seed:
both sides read the same host buffers, so parity does not depend on the
generator being stable across torch versions.

Workloads (sizes and distributions of the pages' examples and of the
throughput studies built on them):

* ``row_shift``: the worked example of "Asynchronous Copies" (section "A
  Global-to-Shared Copy"): a 64x4 float32 tensor holding 0..255 in row-major
  order.
* ``scale2_small``: 2**24 floats uniform in [-1, 1), seed 1; tile 256, 2
  stages, 64 tiles per workgroup ("CUDA Async Copy and Pipeline Guide",
  section "Implementation Comparison": a double-buffered scale-by-2 over
  256-float tiles).
* ``scale2_sweep``: 2**28 floats (1 GiB in, 1 GiB out), seed 2; stages 1..4 x
  tile 256/1024/4096, plus a 4-byte source offset that forces the
  element-wise fallback ("Asynchronous Data Movement", sections "Alignment
  requirements" and "Double buffering"; the guide's FAQ on 2-4 stages).
* ``chunk_copy``: 2**26 16-byte chunks of float32x4 values uniform in [-1, 1),
  seed 3; pred ~ Bernoulli(0.9), src_size uniform on {0, 4, 8, 12, 16}, 1 %
  ignore_src; destination pre-filled with the word 0xDEADBEEF ("Asynchronous
  Copies", paragraph on pred, src_size and ignore_src).
* ``horner32``: 2**27 floats uniform in [-1, 1), seed 4; a 32-step fmaf chain
  per element; tile 1024, stages 1, 2, 4.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

DEADBEEF = 0xDEADBEEF


def uniform_pm1(n: int, seed: int) -> torch.Tensor:
    """n float32 values uniform in [-1, 1) as ``2 * rand - 1``.

    torch's float32 ``rand`` returns multiples of 2**-24 in [0, 1), so doubling
    and subtracting one is exact: the values are multiples of 2**-23 in [-1, 1).
    """
    g = torch.Generator().manual_seed(seed)
    return torch.rand(n, generator=g, dtype=torch.float32).mul_(2.0).sub_(1.0)


def arange_rows(rows: int = 64) -> torch.Tensor:
    """(rows, 4) float32 tensor holding 0 .. 4*rows-1 in row-major order."""
    return torch.arange(rows * 4, dtype=torch.float32).reshape(rows, 4)


def random_rows(rows: int, seed: int) -> torch.Tensor:
    """(rows, 4) float32 tensor of arbitrary 32-bit patterns (NaNs included)."""
    g = torch.Generator().manual_seed(seed)
    bits = torch.randint(-(2 ** 31), 2 ** 31, (rows, 4), generator=g, dtype=torch.int64)
    return bits.to(torch.int32).view(torch.float32)


@dataclass
class ChunkCopyInputs:
    src: torch.Tensor          # uint8 (n_chunks, 16)
    dst_init: torch.Tensor     # uint8 (n_chunks, 16), the pre-filled destination
    pred: torch.Tensor         # uint8 (n_chunks,)
    src_size: torch.Tensor     # uint8 (n_chunks,)
    ignore_src: torch.Tensor   # uint8 (n_chunks,)


def prefill_words(n_words: int, word: int = DEADBEEF) -> torch.Tensor:
    """n_words 32-bit words of ``word`` (little-endian bytes), as int32."""
    signed = word - (1 << 32) if word >= (1 << 31) else word
    return torch.full((n_words,), signed, dtype=torch.int32)


def chunk_copy_inputs(n_chunks: int, seed: int = 3, p_pred: float = 0.9,
                      p_ignore: float = 0.01, sizes=(0, 4, 8, 12, 16)) -> ChunkCopyInputs:
    """Inputs for the predicated chunk copy, drawn in the order values, pred,
    src_size, ignore_src from one generator."""
    g = torch.Generator().manual_seed(seed)
    vals = torch.rand(n_chunks * 4, generator=g, dtype=torch.float32).mul_(2.0).sub_(1.0)
    src = vals.view(torch.uint8).reshape(n_chunks, 16)
    pred = (torch.rand(n_chunks, generator=g) < p_pred).to(torch.uint8)
    size_tab = torch.tensor(sizes, dtype=torch.uint8)
    src_size = size_tab[torch.randint(0, len(sizes), (n_chunks,), generator=g)]
    ignore = (torch.rand(n_chunks, generator=g) < p_ignore).to(torch.uint8)
    dst = prefill_words(n_chunks * 4).view(torch.uint8).reshape(n_chunks, 16)
    return ChunkCopyInputs(src, dst, pred, src_size, ignore)


@dataclass(frozen=True)
class Workload:
    name: str
    op: str
    n: int
    seed: int
    tiles: tuple = ()
    stages: tuple = ()
    tiles_per_block: int = 64
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "row_shift": Workload("row_shift", "row_shift", 64, 0),
    "scale2_small": Workload("scale2_small", "scale2", 1 << 24, 1, (256,), (2,), 64),
    "scale2_sweep": Workload("scale2_sweep", "scale2", 1 << 28, 2, (256, 1024, 4096),
                             (1, 2, 3, 4), 64, {"src_offset_bytes": (0, 4)}),
    "chunk_copy": Workload("chunk_copy", "chunk_copy", 1 << 26, 3, (256,), (2,), 64),
    "horner32": Workload("horner32", "horner32", 1 << 27, 4, (1024,), (1, 2, 4), 64),
}
