"""Static checks of libtilepipe's own gfx950 machine code (no GPU needed).

The kernels issue their memory instructions from inline assembly, which the
compiler's hazard recognizer cannot see into. These checks disassemble the
code object built here and verify the rules those asm blocks must keep:

* every buffer instruction is preceded by at least 5 wait states ("s_nop 4"):
  a VALU write of an SGPR followed by a vector-memory instruction that reads
  it needs 5 (the compiler may rebuild a descriptor with v_readfirstlane right
  before the asm block), and an LDS-DMA load needs 1 after its M0 write;
* every LDS-DMA load has its M0 written inside the same block;
* every 16-byte store is followed by a wait state (store-data hazard);
* no instruction touches memory without a range check (no global_, flat_ or
  scratch_ instructions) and nothing writes through the scalar cache;
* a kernel drains its LDS-DMA loads (vmcnt(0)) before it ends.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from software_pipelining_amd import tilepipe

OBJDUMP = "/opt/rocm/lib/llvm/bin/llvm-objdump"


def _sregs(tok: str):
    m = re.match(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", tok)
    return {int(m.group(1))} if m else set()


@pytest.fixture(scope="module")
def kernels():
    lib = tilepipe.library_path()
    if not os.path.exists(lib):
        pytest.skip("libtilepipe.so is not built")
    if not os.path.exists(OBJDUMP):
        pytest.skip("llvm-objdump not available")
    funcs = {}
    with tempfile.TemporaryDirectory() as d:
        so = os.path.join(d, "lib.so")
        shutil.copy(lib, so)
        subprocess.run([OBJDUMP, "--offloading", so], cwd=d, check=True, capture_output=True)
        objs = [os.path.join(d, f) for f in os.listdir(d) if f.endswith("gfx950")]
        assert objs, "no gfx950 code object in the library"
        for obj in objs:
            out = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", obj], check=True,
                                 capture_output=True, text=True).stdout
            name = None
            for line in out.splitlines():
                m = re.match(r"^[0-9a-f]+ <(.*)>:", line)
                if m:
                    name = m.group(1)
                    funcs[name] = []
                    continue
                m = re.match(r"\s+([a-z_0-9]+)\s*(.*?)\s*//", line)
                if m and name:
                    funcs[name].append((m.group(1), [t.strip() for t in m.group(2).split(",")]))
    return funcs


def test_kernels_present(kernels):
    names = " ".join(kernels)
    for k in ("map_kernel", "chunk_copy_kernel", "row_shift_kernel"):
        assert k in names


def test_buffer_instructions_have_wait_states(kernels):
    n = 0
    for name, insts in kernels.items():
        for i, (op, ops) in enumerate(insts):
            if not op.startswith("buffer_"):
                continue
            n += 1
            prev_op, prev_ops = insts[i - 1]
            assert prev_op == "s_nop" and int(prev_ops[0], 0) >= 4, (name, i, op)
            # and, linearly, no VALU write of an operand SGPR in the 5 wait states
            used = set()
            for t in ops:
                if t:
                    used |= _sregs(t.split()[0])
            ws, j = 0, i - 1
            while j >= 0 and ws < 5:
                pop, pops = insts[j]
                assert not (pop.startswith("v_") and pops and _sregs(pops[0]) & used), (name, i, op)
                ws += int(pops[0], 0) + 1 if pop == "s_nop" else 1
                j -= 1
    assert n > 1000


def test_lds_dma_sets_m0_in_block(kernels):
    for name, insts in kernels.items():
        for i, (op, ops) in enumerate(insts):
            if op.startswith("buffer_load") and "lds" in ops[-1]:
                assert insts[i - 2][0] == "s_mov_b32" and insts[i - 2][1][0] == "m0", (name, i)


def test_wide_stores_followed_by_wait_state(kernels):
    for name, insts in kernels.items():
        for i, (op, _) in enumerate(insts):
            if op in ("buffer_store_dwordx4", "buffer_store_dwordx3"):
                assert insts[i + 1][0] == "s_nop", (name, i)


def test_no_unchecked_or_scalar_memory_writes(kernels):
    for name, insts in kernels.items():
        for op, _ in insts:
            assert not op.startswith(("global_", "flat_", "scratch_")), (name, op)
            assert not op.startswith(("s_store", "s_buffer_store", "s_atomic", "s_buffer_atomic",
                                      "s_dcache_wb", "s_dcache_discard")), (name, op)


def test_lds_dma_drained_before_end(kernels):
    for name, insts in kernels.items():
        last_dma = max((i for i, (op, ops) in enumerate(insts)
                        if op.startswith("buffer_load") and "lds" in ops[-1]), default=None)
        if last_dma is None:
            continue
        ends = [i for i, (op, _) in enumerate(insts) if op == "s_endpgm"]
        assert ends
        for e in ends:
            if e < last_dma:
                continue
            seg = insts[last_dma:e]
            assert any(op == "s_waitcnt" and "vmcnt(0)" in " ".join(ops) for op, ops in seg), name
