"""Static checks of libtilepipe's own gfx950 machine code (no GPU needed).

The kernels issue their memory instructions from inline assembly, which the
compiler's hazard recognizer cannot see into. These checks disassemble the
code object built here and verify the rules those asm blocks must keep:

* every buffer instruction is preceded by at least 5 wait states ("s_nop 4"):
  a VALU write of an SGPR followed by a vector-memory instruction that reads
  it needs 5 (the compiler may rebuild a descriptor with v_readfirstlane right
  before the asm block), and an LDS-DMA load needs 1 after its M0 write;
* every LDS-DMA load has its M0 written inside the same block;
* every 16-byte store is followed by two wait states before a VALU may write
  its data registers (store-data hazard);
* no instruction touches memory without a range check (no global_, flat_ or
  scratch_ instructions) and nothing writes through the scalar cache;
* on every path through a kernel's control flow, each LDS-DMA load has
  retired before s_endpgm (a vmcnt wait small enough that only operations
  issued after the last such load can still be outstanding).
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


def _disassemble():
    """{kernel name: [(op, operands, address, branch target address or None)]}"""
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
            name = base = None
            for line in out.splitlines():
                m = re.match(r"^([0-9a-f]+) <(.*)>:", line)
                if m:
                    base, name = int(m.group(1), 16), m.group(2)
                    funcs[name] = []
                    continue
                m = re.match(r"\s+([a-z_0-9]+)\s*(.*?)\s*// ([0-9A-Fa-f]+):(.*)$", line)
                if m and name:
                    t = re.search(r"<(.*)\+0x([0-9a-f]+)>", m.group(4))
                    target = base + int(t.group(2), 16) if t and t.group(1) == name else None
                    funcs[name].append((m.group(1), [x.strip() for x in m.group(2).split(",")],
                                        int(m.group(3), 16), target))
    return funcs


@pytest.fixture(scope="module")
def disassembly():
    return _disassemble()


@pytest.fixture(scope="module")
def kernels(disassembly):
    return {k: [(op, ops) for op, ops, _, _ in v] for k, v in disassembly.items()}


def test_kernels_present(kernels):
    names = " ".join(kernels)
    for k in ("map_kernel", "chunk_copy_kernel", "row_shift_kernel", "workgroup_copy_kernel",
              "workgroup_copy_clear_kernel"):
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


def test_m0_belongs_to_the_lds_dma_blocks(kernels):
    # The asm blocks write M0 without declaring it (the compiler reserves that
    # register and refuses it in a clobber list). That is only sound while no
    # compiler-generated instruction keeps a value of its own in M0: every
    # mention of M0 must be one of those writes, directly followed by the
    # block's wait states and its LDS-DMA load.
    n = 0
    for name, insts in kernels.items():
        for i, (op, ops) in enumerate(insts):
            if not any(re.search(r"\bm0\b", t) for t in ops):
                continue
            assert op == "s_mov_b32" and ops[0] == "m0", (name, i, op, ops)
            assert insts[i + 1][0] == "s_nop", (name, i)
            nxt_op, nxt_ops = insts[i + 2]
            assert nxt_op.startswith("buffer_load") and "lds" in nxt_ops[-1], (name, i, nxt_op)
            n += 1
    assert n > 1000


def _vregs(tok: str):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def test_wide_stores_followed_by_two_wait_states(kernels):
    # a store of more than 8 bytes reads its data VGPRs late: a VALU write of
    # them needs 2 wait states after it on this architecture family
    n = 0
    for name, insts in kernels.items():
        for i, (op, ops) in enumerate(insts):
            if op not in ("buffer_store_dwordx4", "buffer_store_dwordx3"):
                continue
            n += 1
            nxt_op, nxt_ops = insts[i + 1]
            assert nxt_op == "s_nop" and int(nxt_ops[0], 0) >= 1, (name, i)
    assert n > 1000


def test_wide_store_data_hazard_scan():
    # a rule of the hazard scan itself, checked on known sequences: the two
    # s_nop 0 wait states before a VALU write of the data are counted as two
    seq = [("buffer_store_dwordx4", ["v[4:7]", "v1", "s[0:3]", "0 offen"]),
           ("s_nop", ["0"]), ("v_mov_b32_e32", ["v4", "s3"])]
    assert _store_data_hazards(seq) == [0]
    seq[1] = ("s_nop", ["1"])
    assert _store_data_hazards(seq) == []


def _store_data_hazards(insts):
    """Indices of wide stores whose data VGPRs a VALU writes less than 2 wait
    states later (linear order)."""
    bad = []
    for i, (op, ops) in enumerate(insts):
        if op not in ("buffer_store_dwordx4", "buffer_store_dwordx3"):
            continue
        data, ws = _vregs(ops[0]), 0
        for op2, ops2 in insts[i + 1:i + 4]:
            if ws >= 2:
                break
            if op2 == "s_nop":
                ws += int(ops2[0], 0) + 1
                continue
            if op2.startswith("v_") and ops2 and _vregs(ops2[0].split()[0]) & data:
                bad.append(i)
                break
            ws += 1
    return bad


def test_no_wide_store_data_hazard(kernels):
    for name, insts in kernels.items():
        assert _store_data_hazards(insts) == [], name


def test_no_unchecked_or_scalar_memory_writes(kernels):
    for name, insts in kernels.items():
        for op, _ in insts:
            assert not op.startswith(("global_", "flat_", "scratch_")), (name, op)
            assert not op.startswith(("s_store", "s_buffer_store", "s_atomic", "s_buffer_atomic",
                                      "s_dcache_wb", "s_dcache_discard")), (name, op)


def _is_lds_dma(op, ops):
    return op.startswith("buffer_load") and "lds" in ops[-1]


DRAINED = 1 << 30       # no LDS-DMA load can be outstanding


def _undrained_end(insts):
    """Forward dataflow over one kernel's control-flow graph. The state at an
    instruction is the smallest number, over all paths reaching it, of
    vector-memory operations issued since the last LDS-DMA load (DRAINED once a
    wait has retired every such load). Vector-memory operations of a wave
    retire in issue order, so vmcnt(k) with k not above that number retires
    the load. Returns the index of an s_endpgm reachable with a load in
    flight, else None; the second value counts the s_endpgm visits."""
    index = {addr: i for i, (_, _, addr, _) in enumerate(insts)}
    jumps = _long_jumps(insts)
    state = [None] * len(insts)
    state[0] = DRAINED
    work, ends = [0], 0
    while work:
        i = work.pop()
        op, ops, _, target = insts[i]
        cur = state[i]
        assert not op.startswith("s_swappc"), op
        if op.startswith(("s_setpc", "s_getpc")):
            assert i in jumps or i + 3 in jumps, (i, op)     # only the long-jump pattern
        if _is_lds_dma(op, ops):
            cur = 0
        elif op.startswith("buffer_"):
            cur = cur if cur == DRAINED else cur + 1
        elif op == "s_waitcnt":
            m = re.search(r"vmcnt\((\d+)\)", " ".join(ops))
            if m and int(m.group(1)) <= cur:
                cur = DRAINED
        if op == "s_endpgm":
            ends += 1
            if cur != DRAINED:
                return i, ends
            continue
        succ = []
        if i in jumps:
            assert jumps[i] in index, (i, op)
            state_target = index[jumps[i]]
            new = cur if state[state_target] is None else min(state[state_target], cur)
            if new != state[state_target]:
                state[state_target] = new
                work.append(state_target)
            continue
        if op.startswith(("s_branch", "s_cbranch")):
            assert target is not None and target in index, (i, op)
            succ.append(index[target])
        if op != "s_branch" and i + 1 < len(insts):
            succ.append(i + 1)
        for j in succ:
            new = cur if state[j] is None else min(state[j], cur)
            if new != state[j]:
                state[j] = new
                work.append(j)
    return None, ends


def _long_jumps(insts):
    """{index of s_setpc_b64: target address} for the assembler's long-jump
    sequence  s_getpc_b64 s[a:b]; s_add_u32/s_sub_u32 sa, sa, imm;
    s_addc_u32/s_subb_u32 sb, sb, 0; s_setpc_b64 s[a:b]. s_getpc_b64 yields
    the address of the instruction after it."""
    out = {}
    for i, (op, ops, addr, _) in enumerate(insts):
        if op != "s_getpc_b64" or i + 3 >= len(insts):
            continue
        pair = ops[0]
        lo = "s" + pair[2:pair.index(":")]
        (op1, ops1, _, _), (op2, _, _, _), (op3, ops3, _, _) = insts[i + 1:i + 4]
        assert op1 in ("s_add_u32", "s_sub_u32") and ops1[0] == lo and ops1[1] == lo, (i, op1, ops1)
        assert op2 in ("s_addc_u32", "s_subb_u32") and op3 == "s_setpc_b64" and ops3[0] == pair, (i, op2, op3)
        imm = int(ops1[2], 0)
        out[i + 3] = addr + 4 + (imm if op1 == "s_add_u32" else -imm)
    return out


def _seq(*items):
    """Synthetic instruction list: items are (op, operand string[, target index])."""
    out = []
    for i, it in enumerate(items):
        op, ops = it[0], [x.strip() for x in it[1].split(",")]
        target = 4 * it[2] if len(it) > 2 else None
        out.append((op, ops, 4 * i, target))
    return out


DMA = ("buffer_load_dwordx4", "v1, s[0:3], 0 offen nt lds")
STORE = ("buffer_store_dwordx4", "v[2:5], v1, s[4:7], 0 offen sc1 nt")
END = ("s_endpgm", "")


def test_drain_dataflow_on_known_sequences():
    assert _undrained_end(_seq(DMA, STORE, ("s_waitcnt", "vmcnt(1)"), END))[0] is None
    assert _undrained_end(_seq(DMA, STORE, ("s_waitcnt", "vmcnt(2)"), END))[0] == 3
    assert _undrained_end(_seq(DMA, ("s_waitcnt", "lgkmcnt(0)"), END))[0] == 2
    assert _undrained_end(_seq(DMA, ("s_waitcnt", "vmcnt(0) lgkmcnt(0)"), END))[0] is None
    # a branch around the only wait
    assert _undrained_end(_seq(DMA, ("s_cbranch_scc1", "1", 3), ("s_waitcnt", "vmcnt(0)"),
                               END))[0] == 3
    # two paths: one drained fully then stores, one with a single store; vmcnt(1) covers both
    assert _undrained_end(_seq(DMA, ("s_cbranch_scc1", "1", 5), ("s_waitcnt", "vmcnt(0)"), STORE,
                               ("s_branch", "1", 6), STORE, ("s_waitcnt", "vmcnt(1)"), END))[0] is None
    # a long jump over the only wait (s_getpc_b64 at byte 4 yields 8; 8 + 12 = 20 = index 5)
    assert _undrained_end(_seq(DMA, ("s_getpc_b64", "s[0:1]"), ("s_add_u32", "s0, s0, 12"),
                               ("s_addc_u32", "s1, s1, 0"), ("s_setpc_b64", "s[0:1]"),
                               ("s_waitcnt", "vmcnt(0)"), END))[0] is None
    assert _undrained_end(_seq(DMA, ("s_getpc_b64", "s[0:1]"), ("s_add_u32", "s0, s0, 16"),
                               ("s_addc_u32", "s1, s1, 0"), ("s_setpc_b64", "s[0:1]"),
                               ("s_waitcnt", "vmcnt(0)"), END))[0] == 6
    # a loop whose back edge re-enters after a load with no store behind it
    assert _undrained_end(_seq(STORE, DMA, ("s_cbranch_scc1", "1", 0), ("s_waitcnt", "vmcnt(1)"),
                               END))[0] == 4


def test_lds_dma_drained_before_end(disassembly):
    checked = 0
    for name, insts in disassembly.items():
        bad, ends = _undrained_end(insts)
        assert bad is None, f"{name}: s_endpgm at index {bad} with an LDS-DMA load in flight"
        checked += ends
    assert checked > 100
