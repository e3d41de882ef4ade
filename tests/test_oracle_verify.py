"""Pins of the speculative-verify oracle: all agreement patterns, the
progress guarantee, scaffold auto-accept, and equality with greedy AR decoding
under a deterministic synthetic model."""

import itertools

import numpy as np
import pytest

from oracle import verify as V
from oracle import verify as OV


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


# ---- trajectory-only sampling (Gumbel-max over supplied noise)

def test_gumbel_max_frequencies_follow_softmax():
    # the Gumbel-max construction: argmax(l / T + g), g ~ Gumbel(0, 1), is a
    # draw from softmax(l / T); checked on 200k seeded draws within 5 sigma
    from block_causal_attention_gqa_amd import synth
    l = np.array([1.0, 0.3, -0.5, 2.0, 0.0], np.float32)
    for T in (1.0, 0.7, 2.5):
        n = 200_000
        g = synth.gumbel(3, (n, l.size), int(T * 10))
        pert = OV.perturbed_row(np.broadcast_to(l, (n, l.size)), g, 1.0 / T)
        freq = np.bincount(pert.argmax(axis=1), minlength=l.size) / n
        p = np.exp(l.astype(np.float64) / T)
        p /= p.sum()
        sigma = np.sqrt(p * (1 - p) / n)
        assert np.all(np.abs(freq - p) < 5 * sigma + 1e-12), (T, freq, p)


def test_cold_limit_is_the_argmax():
    from block_causal_attention_gqa_amd import synth
    l = synth.logits(4, 3, 500, 4.0, 0)
    g = synth.gumbel(4, (3, 500), 0)
    for r in range(3):
        assert OV.argmax_lowest(OV.perturbed_row(l[r], g[r], 1e6)) == OV.argmax_lowest(l[r])


def test_perturbed_value_is_rounded_to_float32_before_comparing():
    # l = (1, 1), g = (0, 2^-25): in float32, 1 + 2^-25 rounds to 1, so the
    # two values tie and the lowest index wins; in float64 index 1 would win
    l = np.array([1.0, 1.0], np.float32)
    g = np.array([0.0, 2.0 ** -25], np.float32)
    assert OV.argmax_lowest(OV.perturbed_row(l, g, 1.0)) == 0
    assert np.argmax(l.astype(np.float64) + g.astype(np.float64)) == 1


def test_sampled_verify_uses_the_perturbed_tokens():
    # drafts equal to the perturbed argmax are all accepted; the bonus comes
    # from the perturbed row
    from block_causal_attention_gqa_amd import synth
    S, L, V = 2, 5, 300
    x = synth.logits(6, S * L, V, 4.0, 0).reshape(S, L, V)
    g = synth.gumbel(6, (S, L, V), 0)
    t = np.array([[OV.argmax_lowest(OV.perturbed_row(x[s, i], g[s, i], 0.5)) for i in range(L)] for s in range(S)])
    acc, bon = OV.spec_verify_sampled(x, g, 0.5, t[:, :4].astype(np.int32), None, np.zeros(S, np.int32))
    assert list(acc) == [4, 4] and list(bon) == list(t[:, 4])
