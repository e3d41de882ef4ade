"""The native pipelined decoding scheduler (bc_pipeline_*, host only, no GPU)
against the schedule oracle: driven with the commit counts the oracle's own
unmask takes on the same seeded logits, it must plan the same steps (active
blocks, modes, counts, commits) and so reveal the same tokens; plus its
argument and order errors."""

import numpy as np
import pytest

from oracle import pipeline as OP, unmask as OU
from block_causal_attention_gqa_amd import binding as B, synth


@pytest.fixture(scope="module", autouse=True)
def _lib():
    try:
        B.lib()
    except (RuntimeError, OSError) as e:
        pytest.skip("libbc.so not built: %s" % e)


def _logits_for(seed, sizes, V, frac):
    def f(b, s):
        x = synth.logits(seed, sizes[b], V, 4.0, 700 + b, s)
        synth.plant_peaks(x, seed, frac, 12.0, 700 + b, s)
        return x
    return f


def _drive(sizes, lf, add, act, tau, n_div, window):
    """Run the native schedule, deciding each step with the oracle unmask."""
    pl = B.Pipeline(sizes, window, add, act, n_div)
    masked = [np.ones(n, np.uint8) for n in sizes]
    tokens = [np.full(n, -1, np.int32) for n in sizes]
    trace = []
    while True:
        plan = pl.plan()
        if plan is None:
            break
        active, local, modes, divs, off, row0 = plan
        assert pl.plan() == plan                       # planning twice gives the same plan
        assert row0 == sum(sizes[:active[0]])
        assert off == list(np.concatenate([[0], np.cumsum([sizes[b] for b in active])]))
        lg = np.concatenate([lf(b, s) for b, s in zip(active, local)])
        om = [OU.MODE_FULL if m == B.BC_UNMASK_FULL else OU.MODE_SEMI for m in modes]
        m_out, t_out, nc, _ = OU.unmask_select(lg, off, om, divs, np.float32(tau),
                                               np.concatenate([masked[b] for b in active]),
                                               np.concatenate([tokens[b] for b in active]))
        for j, b in enumerate(active):
            masked[b], tokens[b] = m_out[off[j]:off[j + 1]].copy(), t_out[off[j]:off[j + 1]].copy()
        done = pl.report(nc)
        trace.append(dict(active=active, modes=["full" if m == B.BC_UNMASK_FULL else "semi" for m in modes],
                          n_commit=[int(x) for x in nc], committed=done))
    pl.close()
    return tokens, trace


@pytest.mark.parametrize("sizes,add,act,n_div,window", [
    ([6, 6, 6, 6, 4], 0.3, 0.7, 4, 3),
    ([6, 6, 6, 6, 4], 0.0, 0.5, 4, 2),
    ([5, 7, 3, 6], 1.0, 1.0, 3, 3),                    # no overlap
    (synth.split_sizes(625, 32), 0.5, 0.9, 4, 3),      # the 625-token variant
    (synth.split_sizes(625, 32), 0.25, 0.5, 8, 3),
])
def test_native_schedule_matches_oracle(sizes, add, act, n_div, window):
    lf = _logits_for(3, sizes, 257 if len(sizes) < 10 else 2048, 0.3)
    want_tok, want_trace = OP.pipelined_decode(sizes, lf, add, act, 0.5, n_div, window)
    got_tok, got_trace = _drive(sizes, lf, add, act, 0.5, n_div, window)
    assert got_trace == want_trace
    for a, b in zip(got_tok, want_tok):
        assert np.array_equal(a, b)


def test_native_schedule_hand_worked():
    # the schedule worked out by hand from the rule (ratios equal to add and
    # to act, a join capped by the window), planned by the native state
    # machine
    from tests.test_oracle_pipeline import (HAND_ACT, HAND_ADD, HAND_N, HAND_SIZES, HAND_TAU, HAND_TRACE,
                                            HAND_WINDOW, hand_logits)
    _, trace = _drive(HAND_SIZES, hand_logits, HAND_ADD, HAND_ACT, HAND_TAU, HAND_N, HAND_WINDOW)
    assert trace == HAND_TRACE


def test_argument_and_order_errors():
    with pytest.raises(B.BcError):
        B.Pipeline([4, 0, 3], 3, 0.5, 0.9, 4)          # empty block
    with pytest.raises(B.BcError):
        B.Pipeline([4, 3], 0, 0.5, 0.9, 4)             # window 0
    with pytest.raises(B.BcError):
        B.Pipeline([4, 3], 3, float("nan"), 0.9, 4)
    pl = B.Pipeline([4, 3], 2, 0.5, 0.9, 2)
    with pytest.raises(B.BcError) as e:
        pl.report([1])                                  # no plan yet
    assert e.value.status == B.BC_ERR_ORDER
    plan = pl.plan()
    assert plan[0] == [0] and plan[2] == [B.BC_UNMASK_FULL] and plan[3] == [2]
    with pytest.raises(B.BcError) as e:
        pl.report([5])                                  # more rows than the block holds
    assert e.value.status == B.BC_ERR_ARG
    assert pl.plan() == plan                            # state unchanged
    assert pl.report([4]) == [0]
    assert pl.plan()[0] == [1]
    assert pl.report([3]) == [1]
    assert pl.plan() is None
    pl.close()
