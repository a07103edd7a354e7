"""Copies between workgroups: the kernel bodies under the CPU emulator
(tests/emu). The same bodies the library builds for gfx950 run on host
buffers: every access is checked against the buffers of the call, every LDS
read against the wait that retires its load, and every wave must end with
no load in flight. The emulator runs one workgroup after another, so a launch
order in which a receiver runs before its sender exercises the bounded wait:
the receiver must give up, set the status word and write nothing ("Asynchronous
Copies", section "Copies between CTAs": the receiver waits for the bytes before
reading them). Each word of a chunk travels with a tag in one 8-byte store; the
clearing kernel zeroes the tags first, so only this call's senders can set
them."""
import numpy as np
import pytest

import oracle
from software_pipelining_amd import tilepipe
from tests import emu

CHUNK = 256


def _buffers(n, seed=0):
    rng = np.random.default_rng(seed)
    src = rng.integers(0, 256, n * CHUNK, dtype=np.uint8)
    dst = rng.integers(0, 256, n * CHUNK, dtype=np.uint8)
    ws = np.full(max(1, tilepipe.workgroup_copy_workspace_bytes(n)) if n else 1, 0xAB, np.uint8)
    status = np.array([7], np.int32)
    return src, dst, ws, status


@pytest.mark.parametrize("n", [1, 2, 3, 64, 257, 1000])
def test_matches_oracle(n):
    src, dst, ws, status = _buffers(n, n)
    expected = oracle.workgroup_copy(src, dst)
    for policy in (0, 1, 2, 3):
        d = dst.copy()
        plan = emu.workgroup_copy(src, d, ws, status, policy=policy, seed=policy, lds_base=128 * policy)
        assert plan.grid == n and plan.threads == 64 and plan.lds_bytes == 512
        assert np.array_equal(d, expected), (n, policy)
        assert status[0] == 0


def test_in_place():
    n = 100
    src, _, ws, status = _buffers(n, 5)
    expected = oracle.workgroup_copy(src, src)
    buf = src.copy()
    emu.workgroup_copy(buf, buf, ws, status)
    assert np.array_equal(buf, expected) and status[0] == 0


def test_receivers_before_their_senders_give_up():
    # launch order n-1, ..., 0: every receiver polls a slot whose tags are not
    # set yet; the first gives up after spin_limit polls and sets the status,
    # the others stop at their next look at the status, and no destination
    # chunk is written
    n = 12
    src, dst, ws, status = _buffers(n, 7)
    d = dst.copy()
    emu.workgroup_copy(src, d, ws, status, spin_limit=20, blocks=list(range(n - 1, -1, -1)))
    assert status[0] == 1
    assert np.array_equal(d, dst)


def test_partial_order_writes_what_arrived():
    # order 0, 2, 1, 3: workgroup 2 finds no tagged words from 1 and gives up;
    # 1 and 3 find their senders' words (0 and 2 sent before they received)
    # and write
    n = 4
    src, dst, ws, status = _buffers(n, 9)
    d = dst.copy()
    emu.workgroup_copy(src, d, ws, status, spin_limit=2, blocks=[0, 2, 1, 3])
    assert status[0] == 1
    exp = oracle.workgroup_copy(src, dst).reshape(n, CHUNK)
    got = d.reshape(n, CHUNK)
    assert np.array_equal(got[[0, 1, 3]], exp[[0, 1, 3]])
    assert np.array_equal(got[2], dst.reshape(n, CHUNK)[2])


def _stale_slots(ws, seed):
    # every staging word tagged as sent, with other data: what an earlier
    # call leaves behind
    words = ws.view(np.uint32).reshape(-1, 2)
    words[:, 0] = np.random.default_rng(seed).integers(0, 2**32, len(words), dtype=np.uint32)
    words[:, 1] = 1


def test_status_and_stale_words_are_cleared_by_the_call():
    # staging words tagged by an earlier call and a set status do not leak
    # into the next call
    n = 33
    src, dst, ws, status = _buffers(n, 11)
    _stale_slots(ws, 12)
    status[0] = 1
    d = dst.copy()
    emu.workgroup_copy(src, d, ws, status, blocks=list(range(n)))
    assert status[0] == 0 and np.array_equal(d, oracle.workgroup_copy(src, dst))


def test_stale_words_are_not_taken_for_the_senders():
    # receivers run before their senders over slots full of an earlier call's
    # tagged words: with the tags cleared first they find nothing, give up and
    # write nothing (taking the stale words would write them into dst)
    n = 9
    src, dst, ws, status = _buffers(n, 14)
    _stale_slots(ws, 15)
    d = dst.copy()
    emu.workgroup_copy(src, d, ws, status, spin_limit=9, blocks=list(range(n - 1, -1, -1)))
    assert status[0] == 1
    assert np.array_equal(d, dst)


def test_planted_short_staging_is_reported():
    # the workspace registered 8 bytes short: the clearing kernel's last
    # store falls outside every writable buffer of the call
    n = 8
    src, dst, ws, status = _buffers(n, 13)
    regions = [(src, False), (dst, True), (ws[:-8], True), (status, True)]
    with pytest.raises(emu.EmulationError, match="outside every writable buffer"):
        emu.workgroup_copy(src, dst.copy(), ws, status, regions=regions)


def test_planning_errors():
    n = 10
    src, dst, ws, status = _buffers(n)
    with pytest.raises(ValueError, match="status 1"):          # workspace too short
        emu.workgroup_copy(src, dst, ws[:-1], status)
    with pytest.raises(ValueError, match="status 4"):          # dst overlapping src in part
        emu.workgroup_copy(src[:-CHUNK], src[CHUNK:], ws, status)
