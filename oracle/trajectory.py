"""Shared-prefix fork with scaffold speculative decoding of a whole
trajectory section -- oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What is computed (restated from the Fast-dDrive method summary, sec. 3.2
"Scaffold Speculative Decoding" and sec. 3.3 on shared-prefix rollouts):
  * N rollouts fork from one decoded prefix whose KV they share; each then
    decodes the trajectory section block by block and keeps its own completed
    blocks in a private cache;
  * a block is decoded in rounds.  In a round the MDM head drafts every
    unverified position of the block in one bidirectional pass, then the AR
    head scores the whole block in one causal pass, which gives the AR
    prediction for every position.  Walking from the first unverified
    position, a draft equal to the AR argmax is accepted; at the first
    mismatch the AR argmax is kept instead (the bonus token, so every round
    advances by at least one position) and the later drafts are dropped;
  * a rollout whose block is complete leaves the following rounds; once every
    rollout has completed the block, each commits it to its private cache and
    the next block starts.

Readings where the pages are silent:
  * the draft of a position is the argmax of its draft logits, taken by the
    unmask step at threshold 0 (every masked row is revealed);
  * row i of the AR logits is aligned with position i; with exactly the
    block's rows of AR logits, a round that accepts every remaining draft has
    no bonus;
  * the K/V a rollout commits for a block are those of its last verify pass
    (a stand-in for the model's forward over the completed block).

The per-round model outputs come from callables, so both sides of a parity
test read the same synthetic data:
  draft_logits(b, r, active)            -> float32 [len(active)][R_b][V]
  verify_logits(b, r, active, tokens)   -> float32 [len(active)][R_b][V]
      (``tokens`` [len(active)][R_b] holds each active rollout's verified
      tokens followed by this round's drafts -- what the AR pass reads; the
      synthetic workloads ignore it, the greedy-AR pin uses it)
  verify_kv(b, r, j)                    -> (k, v) [Hkv][R_b][D] of the j-th
      active rollout's verify pass in round r (only when committing)
``active`` lists the rollouts still decoding block b in round r, ascending.
"""

import numpy as np

from . import kvcache as OK, unmask as OU, verify as OV


def fork_trajectory(block_sizes, n_rollouts, draft_logits, verify_logits, verify_kv=None, priv_shape=None):
    """Decode every block for every rollout.

    Returns dict(tokens [N][sum(block_sizes)] int32, trace (one dict per
    round: block, round, active, first (before the round), accept, bonus),
    rounds [per block], and with ``verify_kv`` the private caches:
    priv_k / priv_v lists of [Hkv][rows][D] arrays, one per rollout).
    ``priv_shape`` = (Hkv, D) of the private caches (needed with verify_kv).
    """
    N = n_rollouts
    total = sum(block_sizes)
    tokens = np.full((N, total), -1, np.int32)
    trace, rounds = [], []
    cache = None
    if verify_kv is not None:
        Hkv, D = priv_shape
        empty = np.zeros((N, Hkv, 0, D), np.float32)
        cache = OK.new_cache(empty, empty, [0] * N)
    row0 = 0
    for b, R in enumerate(block_sizes):
        first = np.zeros(N, np.int64)
        blk = np.full((N, R), -1, np.int32)          # verified tokens of the block
        last = {}                                    # rollout -> (round, slot) of its last verify pass
        r = 0
        while (first < R).any():
            active = [s for s in range(N) if first[s] < R]
            d_lg = draft_logits(b, r, active)
            # draft: every unverified position revealed with its argmax
            drafts = np.empty((len(active), R), np.int32)
            for j, s in enumerate(active):
                masked = (np.arange(R) >= first[s]).astype(np.uint8)
                _, t, _, _ = OU.unmask_select(d_lg[j], [0, R], [OU.MODE_SEMI], [1], np.float32(0.0), masked,
                                              blk[s])
                drafts[j] = t
            v_lg = verify_logits(b, r, active, drafts)
            acc, bon = [], []
            for j, s in enumerate(active):
                a, bonus = OV.spec_verify_one(v_lg[j], drafts[j], None, int(first[s]))
                f = int(first[s])
                blk[s, f:f + a] = drafts[j, f:f + a]
                if bonus >= 0:
                    blk[s, f + a] = bonus
                acc.append(int(a))
                bon.append(int(bonus))
                last[s] = (r, j)
            trace.append(dict(block=b, round=r, active=list(active), first=[int(first[s]) for s in active],
                              accept=acc, bonus=bon))
            for j, s in enumerate(active):
                first[s] += acc[j] + (1 if bon[j] >= 0 else 0)
            r += 1
        rounds.append(r)
        tokens[:, row0:row0 + R] = blk
        if cache is not None:
            for s in range(N):
                k, v = verify_kv(b, *last[s])
                OK.commit(cache, s, cache[s][0].shape[1], np.asarray(k), np.asarray(v))
        row0 += R
    out = dict(tokens=tokens, trace=trace, rounds=rounds)
    if cache is not None:
        out["priv_k"] = [c[0] for c in cache]
        out["priv_v"] = [c[1] for c in cache]
    return out
