"""Pins of the pipelined parallel decoding schedule oracle (Fast-dVLA notes,
key design 4): a schedule worked out by hand from the rule, step by step,
with ratios landing exactly on both thresholds and the window capping a
join; a no-overlap setting reduces to plain block-by-block decoding; and an
overlapping run keeps the rules' invariants."""

import numpy as np
import pytest

from oracle import pipeline as OP, unmask as OU
from block_causal_attention_gqa_amd import synth


def _logits_for(seed, sizes, V, frac):
    def f(b, s):
        x = synth.logits(seed, sizes[b], V, 4.0, 700 + b, s)
        synth.plant_peaks(x, seed, frac, 12.0, 700 + b, s)
        return x
    return f


# ---------------------------------------------------------------------------
# A schedule worked out by hand.  Blocks [8, 8, 8], window 2, add 0.5,
# act 0.75, confidence threshold 0.5, n = 8 (a fully active block with no
# row above the threshold reveals ceil(masked / 8) = 1 row).  The logits of
# block b at its s-th active step are built so that the rows listed in
# CONFIDENT[(b, s)] have confidence 1 / (1 + 63 e^-6) ~ 0.865 (above 0.5) and
# every other row about 1/64 with confidence falling with the row index, so a
# fallback reveals the lowest masked row.  Each row's argmax token encodes
# (b, row, s), so the final tokens record the step each row was revealed at.
#
# Step by step, with "exceeds" strict for both ratio thresholds:
#   0: [0 full]            B0 reveals rows 0-3 (4 confident)      r0 = 4/8
#   1: [0 full]            r0 = 0.5 equals add: B1 does not join;
#                          B0 falls back to row 4                  r0 = 5/8
#   2: [0 full, 1 semi]    r0 = 0.625 exceeds add: B1 joins semi;
#                          B0 row 5; B1 reveals its 5 confident rows
#                                                    r0 = 6/8, r1 = 5/8
#   3: [0 full, 1 semi]    r0 = 0.75 equals act: B1 stays semi; B2's
#                          predecessor exceeds add but two blocks are active
#                          (window 2); B0 row 6; B1 has no confident row and,
#                          semi, reveals nothing       r0 = 7/8, r1 = 5/8
#   4: [0 full, 1 full]    r0 = 0.875 exceeds act: B1 full; window still
#                          caps B2; B0 row 7 (complete, committed); B1 falls
#                          back to row 0                          r1 = 6/8
#   5: [1 full, 2 semi]    B1 is the oldest block; r1 = 0.75 exceeds add (B2
#                          joins) and equals act (B2 semi); B1 row 2; B2
#                          reveals its 2 confident rows    r1 = 7/8, r2 = 2/8
#   6: [1 full, 2 full]    r1 = 0.875 exceeds act; B1 row 4 (complete,
#                          committed); B2 falls back to row 0       r2 = 3/8
#   7: [2 full]            B2 reveals its 5 confident rows (complete)
HAND_SIZES, HAND_V = [8, 8, 8], 64
HAND_ADD, HAND_ACT, HAND_TAU, HAND_N, HAND_WINDOW = 0.5, 0.75, 0.5, 8, 2
CONFIDENT = {(0, 0): [0, 1, 2, 3], (1, 0): [1, 3, 5, 6, 7], (2, 0): [6, 7], (2, 2): [1, 2, 3, 4, 5]}
HAND_TRACE = [
    dict(active=[0], modes=["full"], n_commit=[4], committed=[]),
    dict(active=[0], modes=["full"], n_commit=[1], committed=[]),
    dict(active=[0, 1], modes=["full", "semi"], n_commit=[1, 5], committed=[]),
    dict(active=[0, 1], modes=["full", "semi"], n_commit=[1, 0], committed=[]),
    dict(active=[0, 1], modes=["full", "full"], n_commit=[1, 1], committed=[0]),
    dict(active=[1, 2], modes=["full", "semi"], n_commit=[1, 2], committed=[]),
    dict(active=[1, 2], modes=["full", "full"], n_commit=[1, 1], committed=[1]),
    dict(active=[2], modes=["full"], n_commit=[5], committed=[2]),
]
# the local step at which each row is revealed, read off the walk above
REVEALED_AT = {0: [0, 0, 0, 0, 1, 2, 3, 4], 1: [2, 0, 3, 0, 4, 0, 0, 0], 2: [1, 2, 2, 2, 2, 2, 0, 0]}


def hand_token(b, r, s):
    """The argmax token of row r of block b at its s-th active step."""
    return (8 * b + r + 13 * s) % HAND_V


def hand_logits(b, s):
    x = np.zeros((HAND_SIZES[b], HAND_V), np.float32)
    for r in range(HAND_SIZES[b]):
        t = hand_token(b, r, s)
        x[r, t] = 6.0 if r in CONFIDENT.get((b, s), ()) else 0.5 - 0.01 * r
    return x


def test_hand_worked_schedule():
    tokens, trace = OP.pipelined_decode(HAND_SIZES, hand_logits, HAND_ADD, HAND_ACT, HAND_TAU, HAND_N,
                                        HAND_WINDOW)
    assert trace == HAND_TRACE
    for b, at in REVEALED_AT.items():
        assert tokens[b].tolist() == [hand_token(b, r, s) for r, s in enumerate(at)], b


def test_hand_worked_schedule_catches_planted_mistakes(monkeypatch):
    # reading "exceeds" as ">=" lets B1 join at step 1 and turn full at step 3
    monkeypatch.setattr(OP, "exceeds", lambda r, t: r >= t)
    _, trace = OP.pipelined_decode(HAND_SIZES, hand_logits, HAND_ADD, HAND_ACT, HAND_TAU, HAND_N, HAND_WINDOW)
    assert trace[1]["active"] == [0, 1] and trace != HAND_TRACE
    # a join taken one step late (the predecessor's ratio one reveal behind)
    monkeypatch.setattr(OP, "exceeds", lambda r, t: r - 1.0 / 8 > t)
    _, trace = OP.pipelined_decode(HAND_SIZES, hand_logits, HAND_ADD, HAND_ACT, HAND_TAU, HAND_N, HAND_WINDOW)
    assert trace[2]["active"] == [0] and trace != HAND_TRACE
    # a window that does not cap the join would start B2 at step 3
    monkeypatch.undo()
    _, trace = OP.pipelined_decode(HAND_SIZES, hand_logits, HAND_ADD, HAND_ACT, HAND_TAU, HAND_N, 3)
    assert trace[3]["active"] == [0, 1, 2] and trace != HAND_TRACE


def test_hand_worked_confidences():
    # the two confidence levels the schedule rests on, from their closed forms
    c_hi = OU.row_confidence(hand_logits(0, 0)[0])[3]
    assert abs(c_hi - 1.0 / (1.0 + 63.0 * np.exp(-6.0))) < 1e-15 and c_hi > HAND_TAU
    c_lo = OU.row_confidence(hand_logits(0, 1)[7])[3]
    e = np.exp(np.float64(np.float32(0.5 - 0.07)))
    assert abs(c_lo - e / (e + 63.0)) < 1e-15 and c_lo < HAND_TAU


def test_no_overlap_is_sequential_block_decoding():
    # add = act = 1: no ratio exceeds 1, so a block starts only once its
    # predecessor is committed, fully active, as in plain block decoding
    sizes, V, n, tau = [5, 7, 3, 6], 257, 3, 0.5
    lf = _logits_for(1, sizes, V, 0.3)
    tokens, trace = OP.pipelined_decode(sizes, lf, 1.0, 1.0, tau, n, window=3)
    ref, steps = [], 0
    for b, size in enumerate(sizes):
        m, t, s = np.ones(size, np.uint8), np.full(size, -1, np.int32), 0
        while m.any():
            m, t, _, _ = OU.unmask_select(lf(b, s), [0, size], [OU.MODE_FULL], [n], np.float32(tau), m, t)
            s += 1
            steps += 1
        ref.append(t)
    assert len(trace) == steps
    assert all(len(st["active"]) == 1 and st["modes"] == ["full"] for st in trace)
    for a, b in zip(tokens, ref):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("add,act,window", [(0.3, 0.7, 3), (0.0, 0.5, 2), (0.2, 0.2, 4)])
def test_overlapping_schedule_invariants(add, act, window):
    sizes, V, n, tau = [6, 6, 6, 6, 4], 301, 4, 0.5
    lf = _logits_for(2, sizes, V, 0.35)
    tokens, trace = OP.pipelined_decode(sizes, lf, add, act, tau, n, window)
    # every token revealed, each block committed once, in order
    assert all((t >= 0).all() for t in tokens)
    assert [b for st in trace for b in st["committed"]] == list(range(len(sizes)))
    revealed = [0] * len(sizes)
    committed = 0
    first_active = {}
    for k, st in enumerate(trace):
        assert 1 <= len(st["active"]) <= window
        assert st["active"] == list(range(st["active"][0], st["active"][0] + len(st["active"])))
        assert st["active"][0] == committed
        before = list(revealed)            # transitions are decided from these
        for j, b in enumerate(st["active"]):
            if b not in first_active:
                first_active[b] = k
                if b > committed:     # joined behind an active predecessor: its ratio exceeded add
                    assert before[b - 1] / sizes[b - 1] > add
            if st["modes"][j] == "semi":
                assert b > committed and before[b - 1] / sizes[b - 1] <= act
            else:
                assert b == committed or before[b - 1] / sizes[b - 1] > act
            revealed[b] += st["n_commit"][j]
            assert revealed[b] <= sizes[b]
        assert st["modes"][0] == "full"
        committed += len(st["committed"])
        for b in st["committed"]:
            assert revealed[b] == sizes[b]
    assert revealed == sizes


def test_semi_blocks_commit_only_confident_rows():
    # replay one schedule step by step: a semi-active block's commits are
    # exactly its masked rows whose confidence exceeds the threshold
    sizes, V, n, tau = [8, 8, 8], 211, 4, 0.5
    lf = _logits_for(3, sizes, V, 0.4)
    tokens, trace = OP.pipelined_decode(sizes, lf, 0.25, 0.9, tau, n, window=3)
    masked = [np.ones(s, bool) for s in sizes]
    local = [0] * len(sizes)
    saw_semi = False
    for st in trace:
        for j, b in enumerate(st["active"]):
            x = lf(b, local[b])
            conf = np.array([OU.row_confidence(r)[3] for r in x])
            above = int((masked[b] & (conf > np.float64(np.float32(tau)))).sum())
            if st["modes"][j] == "semi":
                saw_semi = True
                assert st["n_commit"][j] == above
            else:
                assert st["n_commit"][j] >= min(above, int(masked[b].sum()))
            local[b] += 1
        # reconstruct the masks from the final tokens' reveal order is not
        # possible; track counts instead
        for j, b in enumerate(st["active"]):
            # reveal the committed count among the masked rows in the oracle's own order
            k = st["n_commit"][j]
            if k:
                x = lf(b, local[b] - 1)
                conf = np.array([OU.row_confidence(r)[3] for r in x])
                idx = [i for i in np.lexsort((np.arange(sizes[b]), -conf)) if masked[b][i]][:k]
                masked[b][idx] = False
    assert saw_semi
    assert not any(m.any() for m in masked)
