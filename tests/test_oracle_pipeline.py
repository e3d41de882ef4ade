"""Pins of the pipelined parallel decoding schedule oracle (Fast-dVLA notes,
key design 4): a no-overlap setting reduces to plain block-by-block
decoding, and an overlapping run keeps the rules' invariants."""

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


def test_no_overlap_is_sequential_block_decoding():
    # add = act = 1: a block joins only once its predecessor is complete, so
    # every step decodes one block, fully active, as in plain block decoding
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
                if b > committed:     # joined behind an active predecessor: its ratio had reached add
                    assert before[b - 1] / sizes[b - 1] >= add
            if st["modes"][j] == "semi":
                assert b > committed and before[b - 1] / sizes[b - 1] < act
            else:
                assert b == committed or before[b - 1] / sizes[b - 1] >= act
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
