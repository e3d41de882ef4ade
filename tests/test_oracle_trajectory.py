"""Pins of the fork + scaffold speculative trajectory oracle (Fast-dDrive
method summary sec. 3.2 "Scaffold Speculative Decoding", sec. 3.3): a round
trace worked out by hand, the equivalence with greedy AR decoding the pages
state for scaffold speculative decoding, one round per block when every draft
agrees, progress of at least one token per round, and which K/V each rollout
commits."""

import numpy as np
import pytest

from oracle import trajectory as OT
from block_causal_attention_gqa_amd import synth


def onehot_rows(tokens, V, hi=3.0):
    """float32 rows whose argmax is tokens[i] (value hi there, 0 elsewhere)."""
    x = np.zeros((len(tokens), V), np.float32)
    x[np.arange(len(tokens)), tokens] = hi
    return x


def test_hand_worked_rounds():
    # Two rollouts, one block of 5 positions, V = 8.  The AR argmax of
    # position i is (i + 1) % 8 for rollout 0 and (i + 2) % 8 for rollout 1.
    #   round 0: rollout 0 drafts [1, 2, 7, 4, 5]: positions 0, 1 accepted,
    #            mismatch at 2, bonus 3 -> verified through position 2;
    #            rollout 1 drafts [2, 3, 4, 5, 6]: all accepted, no bonus row
    #            -> complete, leaves the next round;
    #   round 1: rollout 0 drafts positions 3, 4 as [4, 0]: position 3
    #            accepted, mismatch at 4, bonus 5 -> complete.
    V, R = 8, 5
    ar = {0: [(i + 1) % V for i in range(R)], 1: [(i + 2) % V for i in range(R)]}
    drafts = {(0, 0): [1, 2, 7, 4, 5], (0, 1): [2, 3, 4, 5, 6], (1, 0): [0, 0, 0, 4, 0]}

    def draft_logits(b, r, active):
        return np.stack([onehot_rows(drafts[(r, s)], V) for s in active])

    def verify_logits(b, r, active, tokens):
        return np.stack([onehot_rows(ar[s], V) for s in active])

    out = OT.fork_trajectory([R], 2, draft_logits, verify_logits)
    assert out["rounds"] == [2]
    assert out["trace"] == [
        dict(block=0, round=0, active=[0, 1], first=[0, 0], accept=[2, 5], bonus=[3, -1]),
        dict(block=0, round=1, active=[0], first=[3], accept=[1], bonus=[5]),
    ]
    assert out["tokens"].tolist() == [[1, 2, 3, 4, 5], [2, 3, 4, 5, 6]]


def _greedy_model(seed, V):
    """A deterministic synthetic AR model: the logits of position i of rollout
    s in block b are seeded by (s, b, i) and the block's tokens before i."""
    def logits(s, b, prev):
        key = [s, b, len(prev)] + [int(t) for t in prev]
        return synth.rng(seed, "misc", 9000, *key).standard_normal(V).astype(np.float32)
    return logits


@pytest.mark.parametrize("p_agree", [0.0, 0.5, 0.9])
def test_rounds_reproduce_greedy_ar(p_agree):
    # Scaffold speculative decoding is lossless: whatever the drafts, the
    # tokens equal greedy AR decoding of the verifier (Fast-dDrive sec. 1).
    seed, V, N, sizes = 11, 12, 3, [6, 4, 5]
    model = _greedy_model(seed, V)
    greedy = {}
    for s in range(N):
        for b, R in enumerate(sizes):
            x = []
            for _ in range(R):
                x.append(int(np.argmax(model(s, b, x))))
            greedy[(s, b)] = x

    def draft_logits(b, r, active):
        out = []
        for s in active:
            want = synth.drafts_with_agreement(seed, greedy[(s, b)], p_agree, V, b, r, s)
            out.append(onehot_rows(want, V))
        return np.stack(out)

    def verify_logits(b, r, active, tokens):
        return np.stack([np.stack([model(s, b, list(tokens[j, :i])) for i in range(sizes[b])])
                         for j, s in enumerate(active)])

    out = OT.fork_trajectory(sizes, N, draft_logits, verify_logits)
    for s in range(N):
        assert out["tokens"][s].tolist() == sum((greedy[(s, b)] for b in range(len(sizes))), [])
    for st in out["trace"]:
        # every round moves every active rollout forward by at least one token
        assert all(a + (bo >= 0) >= 1 for a, bo in zip(st["accept"], st["bonus"]))
    if p_agree == 0.0:
        # no draft agrees: one token (the bonus) per round and rollout
        assert out["rounds"] == sizes


def test_full_agreement_takes_one_round_per_block():
    V, N, sizes = 50, 4, [24, 23, 23]
    t = {(s, b): synth.rng(3, "peak", s, b).integers(0, V, size=R).tolist()
         for s in range(N) for b, R in enumerate(sizes)}
    out = OT.fork_trajectory(sizes, N, lambda b, r, act: np.stack([onehot_rows(t[(s, b)], V) for s in act]),
                             lambda b, r, act, tok: np.stack([onehot_rows(t[(s, b)], V) for s in act]))
    assert out["rounds"] == [1, 1, 1]
    assert all(st["accept"] == [sizes[st["block"]]] * N and st["bonus"] == [-1] * N for st in out["trace"])


def test_private_commits_hold_each_rollouts_last_verify_kv():
    # The K/V value encodes (block, round, slot); the private cache of rollout
    # s must be its blocks' K/V from the round it completed each block in,
    # read at its slot among that round's active rollouts, in block order.
    V, N, sizes, Hkv, D = 6, 3, [3, 2], 1, 2
    ar = lambda s, R: [(s + i) % V for i in range(R)]
    # rollout s agrees with the verifier except at position s of every block
    def draft_logits(b, r, active):
        R = sizes[b]
        return np.stack([onehot_rows([(ar(s, R)[i] + (i == s)) % V for i in range(R)], V) for s in active])

    def verify_logits(b, r, active, tokens):
        return np.stack([onehot_rows(ar(s, sizes[b]), V) for s in active])

    def verify_kv(b, r, j):
        val = np.float32(100 * b + 10 * r + j)
        return np.full((Hkv, sizes[b], D), val), np.full((Hkv, sizes[b], D), -val)

    out = OT.fork_trajectory(sizes, N, draft_logits, verify_logits, verify_kv, priv_shape=(Hkv, D))
    # block 0 (3 rows): rollout 0 mismatches at 0 (bonus) then accepts the
    # rest in round 1; rollout 1 accepts 0, bonus at 1, then the rest in
    # round 1; rollout 2 accepts 0-1, bonus at 2: done in round 0.
    # block 1 (2 rows): rollout 0 takes the bonus at 0 and finishes in
    # round 1 (alone); rollout 1 accepts 0 and takes the bonus at 1, the
    # block's last row, in round 0; rollout 2 has no mismatch inside the
    # block and accepts both rows in round 0.
    last = {0: {0: (1, 0), 1: (1, 1), 2: (0, 2)}, 1: {0: (1, 0), 1: (0, 1), 2: (0, 2)}}
    for s in range(N):
        want = np.concatenate([np.full((Hkv, sizes[b], D), np.float32(100 * b + 10 * last[b][s][0] + last[b][s][1]))
                               for b in range(len(sizes))], axis=1)
        assert np.array_equal(out["priv_k"][s], want), s
        assert np.array_equal(out["priv_v"][s], -want), s
    assert [st["active"] for st in out["trace"]] == [[0, 1, 2], [0, 1], [0, 1, 2], [0]]
