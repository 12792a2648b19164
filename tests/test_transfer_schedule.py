"""CPU model of the fixed-reference streaming kernel's transfer schedule
(attn_mfma.hip, attn_stream_fix): which K/V tile transfers each wave issues
in which iteration, the vmcnt value it waits for at each barrier, and which
LDS buffer every transfer lands in.

The kernel issues K tile u into buffer u % NB in iteration u - NB and V tile
u into buffer u % NB in iteration u - NB + 2 (the prologue plays iterations
-NB .. -1); iteration t reads K tile t+1 (scores) and V tile t-1 (P.V).
Transfers of one wave complete in issue order, so "vmcnt(c)" at a barrier
means: everything this wave issued except its last c transfers has landed.
These tests replay that schedule for every tile count and buffer count the
kernel can meet and check, for every wave's transfer counts:

* at each barrier the tiles the iteration reads have landed (the general
  wait count, and the loop-invariant one of the steady-state loop wherever
  that loop runs);
* no transfer is issued into a buffer that an iteration not yet finished
  still reads.

No GPU is involved.
"""
from __future__ import annotations

import pytest


def issued(j, n, NB, kc, vc):
    """Transfers a wave with kc K and vc V transfers per tile issues in
    iteration j (negative j: the prologue)."""
    vk = j + NB - 2
    return (kc if j + NB < n else 0) + (vc if 0 <= vk < n else 0)


def steady_iterations(n, NB):
    """Iterations run by the six-way unrolled steady-state loop (NB == 3
    only): groups t .. t+5 starting at t = 1 while t + 5 + NB < n."""
    out = set()
    if NB != 3:
        return out
    t = 1
    while t + 5 + NB < n:
        out.update(range(t, t + 6))
        t += 6
    return out


def replay(n, NB, kc, vc):
    seq = []  # (kind, tile) in issue order for this wave

    def issue(kind, u):
        seq.extend([(kind, u)] * (kc if kind == "K" else vc))

    def landed(allowed):
        """Tiles all of whose transfers have landed when at most `allowed`
        of this wave's transfers are still in flight."""
        done = seq[:len(seq) - allowed] if allowed else seq
        return {x for x in set(done)
                if done.count(x) == (kc if x[0] == "K" else vc)}

    # buffer -> (kind, tile) currently held and the last iteration reading it
    last_read = {}

    def reader(kind, u):
        return u - 1 if kind == "K" else u + 1  # scores of K u in iteration u-1

    def put(kind, u, t_issue):
        b = (kind, u % NB)
        if b in last_read:
            prev = last_read[b]
            # the previous occupant's last reader must have finished: it ran
            # in an iteration before t_issue (a barrier sits in between)
            assert reader(kind, prev) < t_issue, (n, NB, kind, u, prev, t_issue)
        last_read[b] = u
        issue(kind, u)

    for u in range(NB):  # prologue
        if u < n:
            put("K", u, u - NB)
        if u >= 2 and u - 2 < n:
            put("V", u - 2, u - NB)
    after = issued(-NB, n, NB, kc, vc) - kc + sum(issued(j, n, NB, kc, vc)
                                                   for j in range(1 - NB, 0))
    assert after >= 0
    if kc:
        assert ("K", 0) in landed(after)
    steady = steady_iterations(n, NB)
    later_ss = (NB - 2) * (kc + vc)
    for t in range(n):
        later = sum(issued(j, n, NB, kc, vc) for j in range(t + 2 - NB, t))
        if t in steady:
            assert t + NB < n
            assert later == later_ss, (n, NB, kc, vc, t)
        got = landed(later)
        if t + 1 < n and kc:
            assert ("K", t + 1) in got, (n, NB, kc, vc, t)
        if t >= 1 and vc:
            assert ("V", t - 1) in got, (n, NB, kc, vc, t)
        before = len(seq)
        if t + NB < n:
            put("K", t + NB, t)
        if t + NB - 2 < n:
            put("V", t + NB - 2, t)
        assert len(seq) - before == issued(t, n, NB, kc, vc)
    # the last P.V waits with vmcnt(0): everything has landed
    if vc:
        assert ("V", n - 1) in landed(0)


@pytest.mark.parametrize("NB", [3, 4, 5, 6])
def test_schedule_every_tile_count(NB):
    for n in range(1, 48):
        for kc in range(4):
            for vc in range(4):
                replay(n, NB, kc, vc)


def test_steady_loop_covers_the_middle():
    """For long rows the steady-state loop runs all but a few iterations."""
    n = 64
    s = steady_iterations(n, 3)
    assert min(s) == 1 and max(s) >= n - 9 and len(s) % 6 == 0


def test_model_catches_a_short_wait():
    """One transfer more in flight than the kernel allows leaves part of a
    tile the iteration needs outstanding: the model must see that."""
    n, NB, kc, vc = 10, 3, 2, 1
    seq = []
    for u in range(NB):
        if u < n:
            seq.extend([("K", u)] * kc)
        if u >= 2:
            seq.extend([("V", u - 2)] * vc)
    ok = issued(-1, n, NB, kc, vc)  # the kernel's count at iteration 0
    done_ok = seq[:len(seq) - ok]
    assert done_ok.count(("K", 1)) == kc
    done_bad = seq[:len(seq) - (ok + 1)]
    assert done_bad.count(("K", 1)) < kc
