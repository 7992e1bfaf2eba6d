"""CPU model of the synchronisation protocol of the TTT-Linear / delta-rule matrix-core kernel
(test_sequence_layers_amd/csrc/linear_mfma.hip).

The kernel streams chunks into an LDS ring with direct-to-LDS loads from loader waves and
synchronises every wave with one barrier per group of chunks.  Nothing orders the ring's
LDS traffic except (1) each loader's vmcnt wait before a barrier and (2) the barrier
intervals in which the other waves read a slot or a handoff buffer.  This model replays the
schedule for every chunk count and checks, for every read:
  * the chunk's loads have landed before the barrier that opens the reading interval;
  * no refill of the chunk's slot is issued before the last interval that reads it ends;
and for the handoff and pair-correction buffers that every read sees the write of the
interval before and no later write.  The constants are those of the source, which the
test checks are still there; planted mistakes (a wait one chunk short, an early refill, a
handoff read in the interval it is written) must be caught.
"""
import os
import re

import pytest

SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "test_sequence_layers_amd", "csrc",
                   "linear_mfma.hip")

RING = 24
GROUP = 4


def loads_per_chunk(p, tok):
    """Direct-to-LDS loads per chunk of loader p: Q tile (2) + V half tile (1); K tile (2) +
    rates."""
    return 3 if p == 0 else 2 + (1 if tok else 0)


def clampw(nchunks, per):
    """Outstanding loads allowed by a wait on nchunks chunks (6-bit vmcnt)."""
    return nchunks * per if nchunks * per < 64 else (63 // per) * per


def test_constants_match_the_source():
    src = open(SRC).read()
    assert "static constexpr int kRing = 24;" in src
    assert "constexpr int kGroup = 4;" in src
    assert "static constexpr int kAhead = kDelta ? 2 : 0;" in src
    assert "return p == 0 ? 3 : 2 + (kTok ? 1 : 0);" in src
    assert "kWait0 = clampw(kRing - 2 - kGroup - kAhead, loads(P))" in src
    assert "kWait1 = clampw(kRing - 2 - 2 * kGroup - kAhead, loads(P))" in src
    assert "kWaitN = clampw(kRing - 2 - 3 * kGroup - kAhead, loads(P))" in src
    # refill after barrier b: chunks kGroup b - 2 kGroup + kRing .. + kGroup - 1
    assert "issue(kGroup * b - 2 * kGroup + kRing + x)" in src


def simulate(nchunks, delta, tok, *, wait_short=0, refill_shift=0, handoff_same_interval=False):
    """Replay the schedule; returns a list of violations (empty when the protocol holds)."""
    R, G = RING, GROUP
    ahead = 2 if delta else 0
    ngroups = (nchunks + G - 1) // G
    bad = []
    landed = {}   # (loader, barrier) -> highest chunk index all of whose loads have landed
    refill = {}   # chunk -> barrier after which it is issued (-1: before barrier 0)
    for p in (0, 1):
        L = loads_per_chunk(p, tok)
        issued = list(range(R))              # chunk ids in issue order
        for c in issued:
            refill.setdefault(c, -1)

        def done(allowed):
            k = allowed // L                 # whole chunks still outstanding
            return issued[len(issued) - 1 - k] if k < len(issued) else -1
        w0 = clampw(R - 2 - G - ahead + wait_short, L)
        w1 = clampw(R - 2 - 2 * G - ahead + wait_short, L)
        wn = clampw(R - 2 - 3 * G - ahead + wait_short, L)
        landed[(p, 0)] = done(w0)
        nbar = 1
        if ngroups >= 1:
            landed[(p, 1)] = done(w1)
            nbar += 1
        for b in range(2, ngroups + 1):
            landed[(p, b)] = done(wn)
            nbar += 1
            if b < ngroups:
                for x in range(G):
                    c = G * b - 2 * G + R + x + refill_shift
                    issued.append(c)
                    refill[c] = b
        if nbar != ngroups + 1:
            bad.append(("loader barrier count", p, nbar, ngroups + 1))
    # reads: chunk -> intervals (interval i runs from barrier i to barrier i + 1)
    reads = {}

    def read(c, interval):
        reads.setdefault(c, set()).add(interval)
    read(0, 0)
    read(1, 0)
    for grp in range(ngroups):
        for c in range(G * grp + 2, G * grp + 6):   # chain waves, one pair ahead
            read(c, grp)
        for c in range(G * grp, G * grp + G):       # output waves, one group behind
            read(c, grp + 1)
        if delta and grp + 1 < ngroups:             # Tm waves, the next group
            for c in range(G * (grp + 1), G * (grp + 1) + G):
                read(c, grp)
    for c, ivs in reads.items():
        first, last = min(ivs), max(ivs)
        if first > ngroups:
            continue
        for p in (0, 1):
            if landed.get((p, first), -1) < c:
                bad.append(("not landed", c, first, p))
        # the next chunk issued into c's slot must come after the last reading interval
        for c2, b2 in refill.items():
            if c2 > c and c2 % R == c % R and c2 <= c + R and b2 < last + 1:
                bad.append(("slot overwritten", c, c2, b2, last))
    # handoff buffers (by group parity): chain waves write group grp's in interval grp,
    # output waves read it in interval grp + 1; delta N buffers: the Tm waves write group
    # grp's in interval grp - 1 (group 0 before barrier 0), the chain waves read it in
    # interval grp
    events = []
    for grp in range(ngroups):
        w_iv = grp
        r_iv = grp if handoff_same_interval else grp + 1
        events.append(("hand", grp & 1, w_iv, r_iv))
        if delta:
            events.append(("n", grp & 1, grp - 1, grp))
    for kind, buf, w, r in events:
        if not w < r:
            bad.append(("read before write", kind, buf, w, r))
        for kind2, buf2, w2, _ in events:
            if kind2 == kind and buf2 == buf and w < w2 <= r:
                bad.append(("rewritten before read", kind, buf, w, w2, r))
    return bad


@pytest.mark.parametrize("delta,tok", [(False, False), (False, True), (True, False), (True, True)])
def test_protocol_holds_for_every_chunk_count(delta, tok):
    for nchunks in range(1, 130):
        assert simulate(nchunks, delta, tok) == [], nchunks


@pytest.mark.parametrize("delta", [False, True])
def test_planted_mistakes_are_caught(delta):
    # a wait one chunk short, a refill one chunk early and a handoff read in the interval that
    # writes it must each break the protocol for some chunk count
    assert any(simulate(n, delta, False, wait_short=1) for n in range(1, 80))
    assert any(simulate(n, delta, False, refill_shift=-1) for n in range(1, 80))
    assert any(simulate(n, delta, False, handoff_same_interval=True) for n in range(1, 80))
