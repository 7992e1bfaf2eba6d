"""CPU model of the LDS ring protocols of the TTT-Linear backward kernels
(test_sequence_layers_amd/csrc/linear_bwd_mfma.hip).

Loader waves stream one step's tiles into a ring slot with direct-to-LDS loads; nothing
orders that traffic except each loader's vmcnt wait before a barrier and the barrier
intervals in which the compute waves read a slot.  Two protocols:
  * the state-history kernel reads step s's slot one interval early (operands a step
    ahead in registers): barrier k must publish steps up to k + 1;
  * the reverse kernel's recursion waves read step k's slot in interval k and its gradient
    waves in interval k + 1, through row buffers that alternate between steps.
The model replays each schedule for every chunk count and checks that every read interval
opens after its step's loads have landed, that no refill of a slot is issued before the
last interval reading it has ended, and (reverse kernel) that the gradient waves read the
row buffer written in the interval before and not overwritten until they are done.  The
constants must still be those of the source; planted mistakes must be caught.
"""
import os

import pytest

SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "test_sequence_layers_amd", "csrc",
                   "linear_bwd_mfma.hip")


def test_constants_match_the_source():
    src = open(SRC).read()
    assert "constexpr int kRingF = 8;" in src
    assert "constexpr int kRingB = 6;" in src
    assert "loader_loop_ahead1<kRingF, kTok ? 3 : 2>(nchunks" in src
    assert "loader_loop_lag2<kRingB, kTok ? 5 : 4>(nchunks" in src
    # ahead1: waits R - 2 before barrier 0, R - 3 after; refills step k - 1 + R after barrier k >= 1
    body = src[src.index("void loader_loop_ahead1"):src.index("void loader_loop_ahead1") + 900]
    assert "wait_vmcnt<(R - 2) * kLoads>();" in body and "wait_vmcnt<(R - 3) * kLoads>();" in body
    assert "if (k >= 1) issue(k - 1 + R);" in body and "for (int k = 0; k <= nsteps; ++k)" in body
    # lag2: waits R - 1, R - 2, then R - 3; refills step k - 2 + R after barriers 2 .. nsteps - 1
    body = src[src.index("void loader_loop_lag2"):src.index("void loader_loop_lag2") + 900]
    for w in ("(R - 1)", "(R - 2)", "(R - 3)"):
        assert f"wait_vmcnt<{w} * kLoads>();" in body
    assert "if (k >= 2 && k < nsteps) issue(k - 2 + R);" in body


def _schedule(reads, nbarriers):
    """reads(k) -> steps read in the interval after barrier k; returns it with each step's
    last reading interval."""
    last = {}
    for k in range(nbarriers):
        for s in reads(k):
            last[s] = max(last.get(s, -1), k)
    return last


def _run(R, nbarriers, waits, refill_at, reads):
    """waits(k): steps a loader may leave outstanding before barrier k; refill_at(k): the step
    issued after barrier k (or None); reads(k): the steps read in the interval after barrier
    k.  Loads land in issue order.  Returns the violations."""
    bad = []
    outstanding, landed, owner = [], set(), {}
    last_read = _schedule(reads, nbarriers)

    def issue(s):
        outstanding.append(s)
        owner[s % R] = s

    for s in range(R):
        issue(s)
    for k in range(nbarriers):
        while len(outstanding) > waits(k):
            landed.add(outstanding.pop(0))
        s_new = refill_at(k)
        if s_new is not None:
            old = s_new - R
            if old >= 0 and last_read.get(old, -1) >= k:
                bad.append(("refill before the last read", k, old))
            issue(s_new)
        for s in reads(k):
            if s not in landed:
                bad.append(("read before landing", k, s))
            if owner[s % R] != s:
                bad.append(("slot overwritten", k, s))
    return bad


def ahead1(nsteps, R=8, wait_short=0, refill_shift=0):
    """History kernel: step 0 and 1 read after barrier 0, step k + 1 after barrier k."""
    def reads(k):
        return [0, 1] if k == 0 else ([k + 1] if k < nsteps else [])

    def waits(k):
        return (R - 2 if k == 0 else R - 3) + wait_short

    def refill(k):
        return k - 1 + R + refill_shift if k >= 1 else None
    return _run(R, nsteps + 1, waits, refill, reads)


def lag2(nsteps, R=6, wait_short=0, refill_shift=0):
    """Reverse kernel: recursion waves read step k after barrier k, gradient waves step k - 1."""
    def reads(k):
        r = [k] if k < nsteps else []
        if k >= 1:
            r.append(k - 1)
        return r

    def waits(k):
        return (R - 1 if k == 0 else R - 2 if k == 1 else R - 3) + wait_short

    def refill(k):
        return k - 2 + R + refill_shift if 2 <= k < nsteps else None
    return _run(R, nsteps + 1, waits, refill, reads)


def row_buffers(nsteps, same_parity=False):
    """Reverse kernel: recursion waves write the rows of step k into buffer k % 2 in interval
    k; gradient waves read step k - 1's rows from buffer (k - 1) % 2 in interval k."""
    bad = []
    holder = {}
    for k in range(nsteps + 1):
        if k >= 1:
            b = (k if same_parity else k - 1) % 2
            if holder.get(b) != k - 1:
                bad.append(("rows", k))
        if k < nsteps:
            holder[k % 2] = k  # written during interval k; visible from barrier k + 1
    return bad


@pytest.mark.parametrize("nsteps", list(range(1, 41)) + [128, 513])
def test_protocols_hold_for_every_chunk_count(nsteps):
    assert ahead1(nsteps) == []
    assert lag2(nsteps) == []
    assert row_buffers(nsteps) == []


def test_planted_mistakes_are_caught():
    # a wait one step short (the history kernel with R - 2 everywhere)
    assert any(ahead1(n, wait_short=1) for n in (3, 9, 40))
    assert any(lag2(n, wait_short=1) for n in (3, 9, 40))
    # a refill one barrier early
    assert any(ahead1(n, refill_shift=-1) for n in (9, 40))
    assert any(lag2(n, refill_shift=-1) for n in (9, 40))
    # gradient waves reading the buffer being written
    assert row_buffers(9, same_parity=True)
