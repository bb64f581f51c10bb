"""The decode kernel's load schedule, emulated on the CPU.

decode_kernel (gemm_decode.hpp) gives each wave the K blocks
kb0 + wave + i*NW, i < n_w, of its split, and cycles them through D register
slots: the first D slots are filled up front, full rounds refill every slot
while two more rounds remain, the last full round refills only blocks that
exist, and a remainder consumes what is left.  This test mirrors that control
flow (it must change with the kernel) and checks, over every small
configuration and the ones the library launches, that

  * every load stays inside the wave's K range (so inside the row), also
    when a wave has fewer blocks than slots;
  * the blocks consumed are exactly the wave's blocks, each once, in order.

A schedule that filled the first slots with their own block indices, as an
earlier form did, fails the first check."""
from __future__ import annotations

import pytest


def schedule(KB: int, NW: int, D: int, S: int, split: int, wave: int, clamp_first: bool = True):
    """(loaded blocks, consumed blocks, the wave's blocks) for one wave."""
    KBs = (KB + S - 1) // S
    kb0 = split * KBs if S > 1 else 0
    KBr = max(0, min(KB, kb0 + KBs) - kb0) if S > 1 else KB
    n_w = (KBr - wave + NW - 1) // NW if wave < KBr else 0
    slot = [None] * D
    loads, consumed = [], []

    def load(d, i):
        kb = kb0 + wave + i * NW
        loads.append(kb)
        slot[d] = kb

    if n_w > 0:
        for d in range(D):
            load(d, min(d, n_w - 1) if clamp_first else d)
    i0 = 0
    while i0 + 2 * D <= n_w:
        for d in range(D):
            consumed.append(slot[d])
            load(d, i0 + d + D)
        i0 += D
    if i0 + D <= n_w:
        for d in range(D):
            consumed.append(slot[d])
            if i0 + d + D < n_w:
                load(d, i0 + d + D)
        i0 += D
    for d in range(D - 1):
        if i0 + d < n_w:
            consumed.append(slot[d])
    mine = [kb0 + wave + i * NW for i in range(n_w)]
    return loads, consumed, mine, (kb0, kb0 + KBr)


def violations(KB, NW, D, S, clamp_first=True):
    bad = []
    for split in range(S):
        for wave in range(NW):
            loads, consumed, mine, (lo, hi) = schedule(KB, NW, D, S, split, wave, clamp_first)
            if any(not lo <= kb < hi for kb in loads) or consumed != mine:
                bad.append((split, wave))
    return bad


@pytest.mark.parametrize("S", [1, 2, 4])
@pytest.mark.parametrize("D", [1, 2, 3, 4])
@pytest.mark.parametrize("NW", [1, 4, 8, 16])
def test_schedule_in_range_and_complete(NW, D, S):
    for KB in list(range(1, 70)) + [112, 144, 224]:
        assert not violations(KB, NW, D, S), (KB, NW, D, S)


def test_unclamped_first_slots_read_out_of_range():
    """Without the clamp, a wave with fewer blocks than slots loads past its
    range (e.g. two K blocks over 16 waves with two slots)."""
    assert violations(2, 16, 2, 1, clamp_first=False)
    assert not violations(2, 16, 2, 1)
