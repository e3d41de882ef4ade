"""Pins of the speculative-verify oracle: all agreement patterns, the
progress guarantee, scaffold auto-accept, and equality with greedy AR decoding
under a deterministic synthetic model."""

import itertools

import numpy as np
import pytest

from oracle import verify as V


def _planted(n_rows, vocab, targets, seed=0):
    """Rows whose argmax is targets[i] by construction."""
    x = np.random.default_rng(seed).uniform(-1, 1, (n_rows, vocab)).astype(np.float32)
    for i, t in enumerate(targets):
        x[i, t] = 5.0
    return x


def test_full_agreement_accepts_everything():
    t = [3, 1, 4, 1, 5, 9]
    lg = _planted(7, 12, t + [2])
    acc, bonus = V.spec_verify_one(lg, np.array(t), None, 0)
    assert acc == 6 and bonus == 2
    acc, bonus = V.spec_verify_one(lg[:6], np.array(t), None, 0)
    assert acc == 6 and bonus == -1


def test_mismatch_at_first_still_makes_progress():
    t = [3, 1, 4, 1]
    lg = _planted(4, 12, t)
    acc, bonus = V.spec_verify_one(lg, np.array([0, 1, 4, 1]), None, 0)
    assert acc == 0 and bonus == 3
    acc, bonus = V.spec_verify_one(lg, np.array([3, 1, 0, 1]), None, 2)
    assert acc == 0 and bonus == 4


@pytest.mark.parametrize("m", [1, 4, 10])
def test_every_agreement_pattern(m):
    vocab = 16
    t = list(np.random.default_rng(m).integers(0, vocab, m))
    lg = _planted(m + 1, vocab, t + [7])
    for bits in itertools.product([0, 1], repeat=m):
        draft = np.array([t[i] if bits[i] else (t[i] + 1) % vocab for i in range(m)])
        first_miss = bits.index(0) if 0 in bits else m
        for first in range(0, min(m, 3) + 1):
            acc, bonus = V.spec_verify_one(lg, draft, None, first)
            k = first_miss if first_miss >= first else first + (bits[first:] + (0,)).index(0)
            assert acc == k - first
            assert bonus == (t[k] if k < m else 7)


def test_scaffold_rows_always_pass():
    t = [3, 1, 4, 1, 5]
    lg = _planted(5, 12, t)
    draft = np.array([3, 0, 0, 1, 0])
    fixed = np.array([0, 1, 1, 0, 0], np.uint8)
    acc, bonus = V.spec_verify_one(lg, draft, fixed, 0)
    assert acc == 4 and bonus == 5


def test_argmax_ties_lowest():
    row = np.zeros((1, 6), np.float32)
    row[0, [2, 4]] = 1.0
    assert V.argmax_lowest(row[0]) == 2
    acc, bonus = V.spec_verify_one(row, np.array([4]), None, 0)
    assert acc == 0 and bonus == 2


def _toy_model(prefix_tokens, pos, vocab):
    """Deterministic stand-in for p_AR(. | x_<pos): logits depend only on the
    position and the tokens before it."""
    h = 1469598103934665603
    for tok in list(prefix_tokens[:pos]) + [pos]:
        h = ((h ^ int(tok)) * 1099511628211) % (1 << 64)
    return np.random.default_rng(h).standard_normal(vocab).astype(np.float32)


@pytest.mark.parametrize("seed", range(8))
def test_speculative_rounds_equal_greedy_ar(seed):
    # Scaffold speculative decoding produces exactly the greedy AR output
    # (Fast-dDrive sec. 1, contributions), from any drafts.
    vocab, n = 9, 12
    rng = np.random.default_rng(seed)
    fixed = (rng.random(n) < 0.25).astype(np.uint8)
    scaffold_tok = rng.integers(0, vocab, n)
    # greedy AR: one token at a time, scaffold positions forced
    ar = []
    for i in range(n):
        ar.append(int(scaffold_tok[i]) if fixed[i] else
                  int(np.argmax(_toy_model(ar, i, vocab))))
    # speculative rounds: draft = anything, verify with the AR logits of the
    # current draft, keep accepted + bonus, redraft the rest
    seq = [int(scaffold_tok[i]) if fixed[i] else int(rng.integers(vocab)) for i in range(n)]
    first, rounds = 0, 0
    while first < n:
        lg = np.stack([_toy_model(seq, i, vocab) for i in range(n)])
        acc, bonus = V.spec_verify_one(lg, np.array(seq), fixed, first)
        k = first + acc
        if k < n:
            seq[k] = bonus
            first = k + 1
        else:
            first = n
        for i in range(first, n):
            if not fixed[i]:
                seq[i] = int(rng.integers(vocab))
        rounds += 1
        assert rounds <= n
    assert seq == ar


def test_batched_matches_single():
    rng = np.random.default_rng(5)
    S, m, vocab = 4, 6, 10
    lg = rng.standard_normal((S, m + 1, vocab)).astype(np.float32)
    draft = rng.integers(0, vocab, (S, m))
    fixed = (rng.random((S, m)) < 0.3).astype(np.uint8)
    first = rng.integers(0, m + 1, S)
    acc, bon = V.spec_verify(lg, draft, fixed, first)
    for s in range(S):
        assert (acc[s], bon[s]) == V.spec_verify_one(lg[s], draft[s], fixed[s], int(first[s]))
