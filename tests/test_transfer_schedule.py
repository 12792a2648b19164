"""CPU model of the fixed-reference streaming kernel's transfer schedule
(attn_mfma.hip, attn_stream_fix): which K/V tile transfers each wave issues
at which barrier, the vmcnt value it waits for there, and which LDS buffer
every transfer lands in.

Schedule (NB LDS buffers per operand): K tile u goes to buffer u % NB and V
tile u to buffer u % NB.  Iteration j owns the transfers of K tile j+NB-1
and V tile j+NB-3 (the prologue plays iterations 1-NB .. -1); iteration t
reads K tile t+1 (scores) and V tile t-1 (P.V) in its block.  A general
iteration waits at its own barrier and issues its own transfers after its
block.  In the steady-state loop a barrier serves a pair of iterations
(t, t+1): it waits for the tiles both blocks read, and each iteration of the
pair issues its transfers after its block.  Either way a transfer is issued
after the last barrier before it and before the next one, which is all the
model below depends on.
Transfers of one wave complete in issue order, so "vmcnt(c)" at a barrier
means: everything this wave issued except its last c transfers has landed.

These tests replay the schedule for every tile count and buffer count the
kernel can meet, for every per-wave transfer count, and check that

* at each barrier the tiles the following block(s) read have landed (the
  general wait count, and the loop-invariant one of the steady-state loop
  wherever that loop runs);
* no transfer is issued into a buffer whose previous tile a block at or
  after that barrier still reads.

No GPU is involved.
"""
from __future__ import annotations

import pytest


def issued(j, n, NB, kc, vc):
    """Transfers a wave with kc K and vc V transfers per tile issues for
    iteration j (negative j: the prologue)."""
    uk, uv = j + NB - 1, j + NB - 3
    return (kc if 0 <= uk < n else 0) + (vc if 0 <= uv < n else 0)


def steady_pairs(n, NB):
    """First iterations of the pairs run by the six-way unrolled steady-state
    loop (NB == 6): groups t .. t+5 starting at t = 1 while t + 5 + NB < n,
    pairs starting at t, t+2, t+4."""
    out = set()
    if NB != 6:
        return out
    t = 1
    while t + 5 + NB < n:
        out.update((t, t + 2, t + 4))
        t += 6
    return out


def wait_general(t, n, NB, kc, vc):
    return sum(issued(j, n, NB, kc, vc) for j in range(t + 3 - NB, t))


def wait_pair(t, n, NB, kc, vc):
    return sum(issued(j, n, NB, kc, vc) for j in range(t + 4 - NB, t))


def replay(n, NB, kc, vc):
    seq = []  # (kind, tile) in issue order for this wave

    def landed(allowed):
        done = seq[:len(seq) - allowed] if allowed else seq
        return {x for x in set(done)
                if done.count(x) == (kc if x[0] == "K" else vc)}

    occupant = {}  # buffer -> tile it holds

    def reader(kind, u):
        return u - 1 if kind == "K" else u + 1  # the block that reads tile u

    def put(kind, u, barrier):
        """Issue tile u at the barrier before block `barrier`."""
        b = (kind, u % NB)
        if b in occupant:
            # the previous tile's reader ran before this barrier
            assert reader(kind, occupant[b]) < barrier, (n, NB, kind, u, occupant[b], barrier)
        occupant[b] = u
        seq.extend([(kind, u)] * (kc if kind == "K" else vc))

    def issue_iteration(j, barrier):
        before = len(seq)
        if 0 <= j + NB - 1 < n:
            put("K", j + NB - 1, barrier)
        if 0 <= j + NB - 3 < n:
            put("V", j + NB - 3, barrier)
        assert len(seq) - before == issued(j, n, NB, kc, vc)

    for j in range(1 - NB, 0):  # prologue (before block 0)
        issue_iteration(j, 0)
    after = issued(1 - NB, n, NB, kc, vc) - kc + sum(issued(j, n, NB, kc, vc)
                                                      for j in range(2 - NB, 0))
    assert after >= 0
    if kc:
        assert ("K", 0) in landed(after)

    pairs = steady_pairs(n, NB)
    ss = (NB - 4) * (kc + vc)  # the steady-state loop's loop-invariant count
    t = 0
    while t < n:
        if t in pairs:
            assert t + 1 + NB - 1 < n          # every transfer of the pair is issued
            w = wait_pair(t, n, NB, kc, vc)
            assert w == ss, (n, NB, kc, vc, t)
            got = landed(w)
            for blk in (t, t + 1):
                if kc and blk + 1 < n:
                    assert ("K", blk + 1) in got, (n, NB, kc, vc, t, blk)
                if vc and blk >= 1:
                    assert ("V", blk - 1) in got, (n, NB, kc, vc, t, blk)
            issue_iteration(t, t)
            issue_iteration(t + 1, t)
            t += 2
        else:
            got = landed(wait_general(t, n, NB, kc, vc))
            if kc and t + 1 < n:
                assert ("K", t + 1) in got, (n, NB, kc, vc, t)
            if vc and t >= 1:
                assert ("V", t - 1) in got, (n, NB, kc, vc, t)
            issue_iteration(t, t)
            t += 1
    # the last P.V waits with vmcnt(0): everything has landed
    if vc:
        assert ("V", n - 1) in landed(0)


@pytest.mark.parametrize("NB", [4, 5, 6])
def test_schedule_every_tile_count(NB):
    for n in range(1, 48):
        for kc in range(4):
            for vc in range(4):
                replay(n, NB, kc, vc)


def test_steady_loop_covers_the_middle():
    """For long rows the steady-state pairs cover all but a few iterations."""
    n = 64
    p = steady_pairs(n, 6)
    covered = set()
    for t in p:
        covered.update((t, t + 1))
    assert min(covered) == 1 and max(covered) >= n - 13 and len(covered) % 6 == 0


def test_model_catches_a_short_wait():
    """One transfer more in flight than the kernel allows at a steady-state
    pair barrier leaves part of a tile a block needs outstanding."""
    n, NB, kc, vc = 40, 6, 2, 1
    seq = []
    for j in range(1 - NB, 7):          # transfers issued before the pair at t = 7
        for u, kind in ((j + NB - 1, "K"), (j + NB - 3, "V")):
            if 0 <= u < n:
                seq.extend([(kind, u)] * (kc if kind == "K" else vc))
    ok = wait_pair(7, n, NB, kc, vc)
    assert seq[:len(seq) - ok].count(("K", 9)) == kc
    assert seq[:len(seq) - (ok + 1)].count(("V", 7)) < vc


def test_model_catches_an_early_overwrite():
    """Issuing the second iteration of a pair into its own K buffer one tile
    earlier (K tile t+NB instead of t+NB-1 ahead) would overwrite the K tile
    block t reads: the buffer check must fire."""
    n, NB = 30, 6
    occupant = {}
    reads_k = {t: t + 1 for t in range(n)}
    bad = False
    t = 7
    for j in (t, t + 1):
        u = j + NB          # one too far
        b = u % NB
        if any(reads_k[blk] % NB == b for blk in (t, t + 1)):
            bad = True
    assert bad
