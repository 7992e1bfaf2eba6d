"""CPU model of the hand-off between the two workgroups of a sequence in the two-workgroup
causal TTT-MLP kernel (mlp_split_kernel in test_sequence_layers_amd/csrc/mlp_mfma.hip).

Every wave of the recursion workgroup stores its update operands of chunk c at the top of
chunk c + 1, before that chunk's prefetch loads, and waits before the first barrier of each
chunk until at most kTopOps of its vector-memory operations are outstanding; operations
complete in issue order.  After that barrier wave 0 publishes a count of complete chunks,
and the output workgroup loads chunk c + 1's operands in its chunk c only once the
published count covers chunk c + 1.  This model replays each wave's operation stream for
every chunk count and both load counts of the prefetch (11, or 12 and 13 with the paper
model's extra load and per-token rates), and checks that:
  * every count published is covered by complete stores of every wave;
  * the output workgroup never loads a chunk that the count it waited for does not cover;
  * the last count (after the final vmcnt(0) and barrier) is the chunk count.
The constants are those of the source, which the test checks are still there; planted
mistakes (a wait that leaves too many operations outstanding, a count one chunk early, an
output workgroup that waits for one chunk too few) must be caught.
"""
import os
import re

import pytest

SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "test_sequence_layers_amd", "csrc",
                   "mlp_mfma.hip")

TOP_OPS = 13  # the wait before the first barrier: at most 13 operations outstanding
WAVES = 8


def _split_source():
    src = open(SRC).read()
    i = src.index("constexpr int kSlotBytes")
    return src, src[i:]


def test_constants_match_the_source():
    src, split = _split_source()
    assert "constexpr int kTopOps = 13;" in src
    assert "__builtin_amdgcn_s_waitcnt(0x0F70 | kTopOps);" in split
    # the progress published after the first barrier of chunk c covers chunks < c - 1
    assert "if (c >= 2) progress(c - 1);" in split
    # the output workgroup, in chunk c, waits for min(c + 2, nchunks) chunks, then loads c + 1
    assert "wait_for(c + 2 < nchunks ? c + 2 : nchunks);" in split
    assert "load_hand<kPaper>(hn, rs, c + 1, wv, lane);" in split
    # stores of the previous chunk come first at the top of a chunk, then the prefetch
    step = split[split.index("auto step = [&](const MainIn& cur, MainIn& nxt, int c) {"):]
    assert step.index("publish(c);") < step.index("load_main<kPaper>(nxt")
    # 2 operand stores per wave (wave 0: 4), 11 unconditional prefetch loads: K rows (2), the
    # K^T gathers (4 x 2), V (1); the paper model's K row and the rate factor are extra
    pub = split[split.index("auto publish = [&](int c) {"):split.index("auto step = [&]")]
    assert pub.count("*reinterpret_cast<u32x4*>(slot") == 4 and "if (wv == 0)" in pub
    lm = split[split.index("__device__ __forceinline__ void load_main"):split.index("struct PartIn")]
    assert lm.count("r.ka0 = __builtin_amdgcn_raw_buffer_load_b128") == 1
    assert lm.count("r.ka1 = __builtin_amdgcn_raw_buffer_load_b128") == 1
    assert "for (int e = 0; e < 4; ++e)" in lm and lm.count("r.kt[e][") == 2
    assert "r.vv = __builtin_amdgcn_raw_buffer_load_b32" in lm
    # the final publication waits for every operation and a barrier
    assert re.search(r"publish\(nchunks\);\s*__builtin_amdgcn_s_waitcnt\(0x0F70\);.*?\n\s*barrier\(\);",
                     split, re.S)


def simulate(nchunks, loads, *, top_ops=TOP_OPS, publish_lag=1, need_ahead=2):
    """Replay the recursion's waves and the output workgroup's reads; returns violations.

    loads: prefetch loads per chunk; publish_lag: the count published in chunk c is
    c - publish_lag; need_ahead: the output workgroup waits for c + need_ahead chunks."""
    bad = []
    # per wave: issue-ordered list of ("store", chunk) / ("load", chunk) / ("poll", c)
    complete_upto = {}   # (wave, chunk c) -> stored chunks complete after the wait of chunk c
    for w in range(WAVES):
        ops = [("load", 0)] * loads            # the first chunk's loads, before the loop
        for c in range(nchunks):
            if c >= 1:
                ops += [("store", c - 1)] * (4 if w == 0 else 2)
            ops += [("load", c + 1)] * loads
            # the wait before the first barrier: all but the newest top_ops complete
            done = ops[:max(0, len(ops) - top_ops)]
            k = 0                                # chunks 0 .. k - 1: every store complete
            while k < c and done.count(("store", k)) == ops.count(("store", k)):
                k += 1
            complete_upto[(w, c)] = k
            if w == 0 and c >= 1:
                ops += [("poll", c)]             # wave 0 reads the partner's word
    published = {}
    for c in range(nchunks):
        if c >= 2:
            count = c - publish_lag
            have = min(complete_upto[(w, c)] for w in range(WAVES))
            if count > have:
                bad.append(("count ahead of stores", c, count, have))
            published[c] = count
    final = nchunks                              # after vmcnt(0) and a barrier
    # the output workgroup: in chunk c it needs the count to cover chunk c + 1
    counts = sorted(published.values()) + [final]
    for c in range(nchunks):
        need = min(c + need_ahead, nchunks)
        got = next(x for x in counts if x >= need)  # the first count that satisfies the wait
        if c + 1 < nchunks and not (c + 1 < got):
            bad.append(("reads an uncovered chunk", c, got))
    return bad


@pytest.mark.parametrize("loads", [11, 12, 13])
def test_protocol_holds_for_every_chunk_count(loads):
    for n in range(1, 70):
        assert simulate(n, loads) == [], (n, loads)


def test_model_catches_a_wait_that_leaves_too_many_operations_outstanding():
    # 26 outstanding operations may still include the stores of chunk c - 2
    assert any(simulate(n, 11, top_ops=26) for n in range(3, 40))


def test_model_catches_a_count_published_one_chunk_early():
    assert any(simulate(n, 11, publish_lag=0) for n in range(3, 40))


def test_model_catches_an_output_workgroup_that_waits_for_one_chunk_too_few():
    assert any(simulate(n, 11, need_ahead=1) for n in range(3, 40))
