"""Pins of the attention oracle against facts other than its own formula.

The mask is pinned by closed forms whose expected visible sets are written out
by hand from the pages' statement of block-causal attention; softmax, scale and
the query-head -> KV-head map are pinned by torch's CPU
scaled_dot_product_attention (an independent library routine) in float64; the
cache is pinned by the cache-free full-sequence recompute; B = 1 is pinned to
causal decoding.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as A


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _sdpa(q, k, v, mask, scale):
    """torch float64 reference: q [R][Hq][D], k/v [L][Hkv][D], mask [R][L]."""
    Hq, Hkv = q.shape[1], k.shape[1]
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))
    kt = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))
    vt = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))
    kt = kt.repeat_interleave(Hq // Hkv, dim=0)
    vt = vt.repeat_interleave(Hq // Hkv, dim=0)
    m = torch.from_numpy(mask)[None].expand(Hq, -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(
        qt[None], kt[None], vt[None], attn_mask=m[None], scale=scale)[0]
    return o.numpy().transpose(1, 0, 2)


def _one_seq(R, Hq, Hkv, D, lp, seed):
    q = _rand((1, R, Hq, D), seed)
    pk = _rand((1, Hkv, lp + 3, D), seed + 1)
    pv = _rand((1, Hkv, lp + 3, D), seed + 2)
    ak = _rand((1, Hkv, R, D), seed + 3)
    av = _rand((1, Hkv, R, D), seed + 4)
    return q, pk, pv, ak, av


# --- closed form: q = 0 gives the plain mean of the visible values ----------

# Hand-written visibility for a prefix of 2 keys and active blocks
# [0,3) [3,5) [5,6): key ids 0,1 = prefix, 2.. = active rows 0..5.
_PREFIX = 2
_BLK_OFF = [0, 3, 5, 6]
_VISIBLE_BIDIR = {
    0: [0, 1, 2, 3, 4], 1: [0, 1, 2, 3, 4], 2: [0, 1, 2, 3, 4],
    3: [0, 1, 2, 3, 4, 5, 6], 4: [0, 1, 2, 3, 4, 5, 6],
    5: [0, 1, 2, 3, 4, 5, 6, 7],
}
_VISIBLE_CAUSAL = {
    0: [0, 1, 2], 1: [0, 1, 2, 3], 2: [0, 1, 2, 3, 4],
    3: [0, 1, 2, 3, 4, 5], 4: [0, 1, 2, 3, 4, 5, 6], 5: [0, 1, 2, 3, 4, 5, 6, 7],
}


@pytest.mark.parametrize("mode,expect", [(A.MASK_BIDIR, _VISIBLE_BIDIR),
                                         (A.MASK_CAUSAL, _VISIBLE_CAUSAL)])
def test_zero_query_averages_exactly_the_visible_keys(mode, expect):
    R, L, D = 6, _PREFIX + 6, 8
    q = np.zeros((1, R, 2, D))
    # value of key id j is the indicator vector e_j, so out[i] reveals the set
    eye = np.eye(D)[:L]
    pk = np.zeros((1, 1, 4, D)); pv = np.zeros((1, 1, 4, D))
    pv[0, 0, :_PREFIX] = eye[:_PREFIX]
    ak = _rand((1, 1, R, D), 5)
    av = eye[_PREFIX:][None, None]
    out = A.attention_step(q, pk, pv, [_PREFIX], ak, av, _BLK_OFF, mode, scale=0.3)
    for i in range(R):
        want = np.zeros(D)
        want[expect[i]] = 1.0 / len(expect[i])
        for h in range(2):
            np.testing.assert_allclose(out[0, i, h], want, atol=1e-15)


def test_single_dominant_key_is_copied():
    # one visible key with a score of +60 above the rest takes all the weight;
    # the same key placed in a later block (invisible) must take none.
    D = 4
    q = np.zeros((1, 2, 1, D)); q[0, :, 0, 0] = 1.0
    pk = np.zeros((1, 1, 3, D)); pv = _rand((1, 1, 3, D), 1)
    ak = np.zeros((1, 1, 2, D)); av = _rand((1, 1, 2, D), 2)
    ak[0, 0, 1, 0] = 60.0          # active row 1 (block 1) is the loud key
    out = A.attention_step(q, pk, pv, [3], ak, av, [0, 1, 2], A.MASK_BIDIR, scale=1.0)
    np.testing.assert_allclose(out[0, 1, 0], av[0, 0, 1], atol=1e-20)
    # row 0 (block 0) cannot see it: plain mean over prefix + itself
    np.testing.assert_allclose(out[0, 0, 0], (pv[0, 0].sum(0) + av[0, 0, 0]) / 4, atol=1e-14)


# --- library cross-check: softmax, scale and the GQA head map ---------------

@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (4, 1), (8, 2), (6, 3)])
@pytest.mark.parametrize("mode", [A.MASK_BIDIR, A.MASK_CAUSAL])
def test_matches_torch_sdpa(Hq, Hkv, mode):
    R, D, lp = 7, 16, 11
    q, pk, pv, ak, av = _one_seq(R, Hq, Hkv, D, lp, 10 * Hq + Hkv)
    blk_off = [0, 2, 5, 7]
    scale = 0.37
    out = A.attention_step(q, pk, pv, [lp], ak, av, blk_off, mode, scale=scale)
    keys = np.concatenate([pk[0, :, :lp], ak[0]], axis=1).transpose(1, 0, 2)
    vals = np.concatenate([pv[0, :, :lp], av[0]], axis=1).transpose(1, 0, 2)
    # visibility written independently: row i of block b may read key j of
    # block c when c < b, or c == b and (bidirectional or j <= i)
    blk = [0, 0, 1, 1, 1, 2, 2]
    mask = np.ones((R, lp + R), dtype=bool)
    for i in range(R):
        for j in range(R):
            ok = blk[j] < blk[i] or (blk[j] == blk[i] and (mode == A.MASK_BIDIR or j <= i))
            mask[i, lp + j] = ok
    ref = _sdpa(q[0], keys, vals, mask, scale)
    np.testing.assert_allclose(out[0], ref, rtol=1e-12, atol=1e-12)


def test_scalar_brute_force_tiny():
    R, Hq, Hkv, D, lp = 3, 2, 1, 3, 2
    q, pk, pv, ak, av = _one_seq(R, Hq, Hkv, D, lp, 99)
    blk_off = [0, 1, 3]
    out = A.attention_step(q, pk, pv, [lp], ak, av, blk_off, A.MASK_BIDIR, scale=0.5)
    blk = [0, 1, 1]
    for i in range(R):
        for h in range(Hq):
            keys, vals = [], []
            for j in range(lp):
                keys.append(pk[0, 0, j]); vals.append(pv[0, 0, j])
            for j in range(R):
                if blk[j] <= blk[i]:
                    keys.append(ak[0, 0, j]); vals.append(av[0, 0, j])
            scores = [0.5 * sum(q[0, i, h, d] * kk[d] for d in range(D)) for kk in keys]
            top = max(scores)
            w = [math.exp(s - top) for s in scores]
            tot = sum(w)
            for d in range(D):
                want = sum(w[n] * vals[n][d] for n in range(len(w))) / tot
                assert abs(out[0, i, h, d] - want) < 1e-13


# --- invariants the pages state ---------------------------------------------

def test_block_size_one_is_causal_decoding():
    # WAM-Diff2 sec. 2.1: B = 1 is standard autoregressive decoding.  With
    # blocks of one token, row i must equal plain unmasked attention of q_i
    # over prefix + active rows 0..i (library SDPA, one row at a time).
    R, Hq, Hkv, D, lp = 6, 4, 2, 8, 5
    q, pk, pv, ak, av = _one_seq(R, Hq, Hkv, D, lp, 3)
    out_b1 = A.attention_step(q, pk, pv, [lp], ak, av, list(range(R + 1)), A.MASK_BIDIR, scale=0.25)
    out_c = A.attention_step(q, pk, pv, [lp], ak, av, [0, R], A.MASK_CAUSAL, scale=0.25)
    np.testing.assert_allclose(out_b1, out_c, rtol=0, atol=1e-15)
    for i in range(R):
        keys = np.concatenate([pk[0, :, :lp], ak[0, :, :i + 1]], axis=1).transpose(1, 0, 2)
        vals = np.concatenate([pv[0, :, :lp], av[0, :, :i + 1]], axis=1).transpose(1, 0, 2)
        ref = _sdpa(q[0, i:i + 1], keys, vals, np.ones((1, lp + i + 1), bool), 0.25)
        np.testing.assert_allclose(out_b1[0, i:i + 1], ref, rtol=1e-12, atol=1e-12)


def test_one_block_is_full_bidirectional_attention():
    R, Hq, Hkv, D, lp = 9, 4, 1, 8, 6
    q, pk, pv, ak, av = _one_seq(R, Hq, Hkv, D, lp, 4)
    out = A.attention_step(q, pk, pv, [lp], ak, av, [0, R], A.MASK_BIDIR, scale=0.3)
    keys = np.concatenate([pk[0, :, :lp], ak[0]], axis=1).transpose(1, 0, 2)
    vals = np.concatenate([pv[0, :, :lp], av[0]], axis=1).transpose(1, 0, 2)
    ref = _sdpa(q[0], keys, vals, np.ones((R, lp + R), bool), 0.3)
    np.testing.assert_allclose(out[0], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("mode", [A.MASK_BIDIR, A.MASK_CAUSAL])
def test_cached_prefix_equals_full_recompute(mode):
    # KV reuse: attending to the cached prefix (two committed blocks plus the
    # prompt) equals recomputing the whole sequence under the block mask.
    Hq, Hkv, D = 4, 2, 8
    prompt, done_blocks, active = 5, [3, 4], [0, 4, 6]
    lp = prompt + sum(done_blocks)
    R = active[-1]
    N = lp + R
    rng = np.random.default_rng(7)
    q_all = rng.standard_normal((N, Hq, D))
    k_all = rng.standard_normal((N, Hkv, D))
    v_all = rng.standard_normal((N, Hkv, D))
    blk = [0] * prompt + [1] * 3 + [2] * 4 + [3] * 4 + [4] * 2
    full = A.full_sequence_attention(q_all, k_all, v_all, blk, mode, scale=0.4)
    pk = k_all[:lp].transpose(1, 0, 2)[None]
    pv = v_all[:lp].transpose(1, 0, 2)[None]
    ak = k_all[lp:].transpose(1, 0, 2)[None]
    av = v_all[lp:].transpose(1, 0, 2)[None]
    out = A.attention_step(q_all[lp:][None], pk, pv, [lp], ak, av, active, mode, scale=0.4)
    np.testing.assert_allclose(out[0], full[lp:], rtol=1e-12, atol=1e-12)


def test_completed_blocks_unaffected_by_later_blocks():
    R, Hq, Hkv, D, lp = 10, 4, 2, 8, 7
    q, pk, pv, ak, av = _one_seq(R, Hq, Hkv, D, lp, 8)
    blk_off = [0, 3, 7, 10]
    before = A.attention_step(q, pk, pv, [lp], ak, av, blk_off, A.MASK_BIDIR)
    q2, ak2, av2 = q.copy(), ak.copy(), av.copy()
    rng = np.random.default_rng(1)
    q2[0, 7:] = rng.standard_normal(q2[0, 7:].shape)
    ak2[0, :, 7:] = rng.standard_normal(ak2[0, :, 7:].shape)
    av2[0, :, 7:] = rng.standard_normal(av2[0, :, 7:].shape)
    after = A.attention_step(q2, pk, pv, [lp], ak2, av2, blk_off, A.MASK_BIDIR)
    assert np.array_equal(before[0, :7], after[0, :7])
    assert not np.allclose(before[0, 7:], after[0, 7:])


def test_fork_equals_independent_runs():
    # Shared-prefix fork: each rollout equals a run whose own cache holds a
    # copy of the shared prefix followed by its private blocks.
    S, R, Hq, Hkv, D = 3, 5, 4, 2, 8
    lp, priv = 9, [0, 4, 2]
    rng = np.random.default_rng(11)
    q = rng.standard_normal((S, R, Hq, D))
    shk = rng.standard_normal((1, Hkv, lp, D)); shv = rng.standard_normal((1, Hkv, lp, D))
    pk = rng.standard_normal((S, Hkv, 6, D)); pv = rng.standard_normal((S, Hkv, 6, D))
    ak = rng.standard_normal((S, Hkv, R, D)); av = rng.standard_normal((S, Hkv, R, D))
    blk_off = [0, 2, 5]
    fork = A.attention_step(q, shk, shv, [lp], ak, av, blk_off, A.MASK_CAUSAL,
                            priv_k=pk, priv_v=pv, priv_len=priv)
    for s in range(S):
        ck = np.concatenate([shk[0], pk[s, :, :priv[s]]], axis=1)[None]
        cv = np.concatenate([shv[0], pv[s, :, :priv[s]]], axis=1)[None]
        solo = A.attention_step(q[s:s + 1], ck, cv, [lp + priv[s]], ak[s:s + 1], av[s:s + 1],
                                blk_off, A.MASK_CAUSAL)
        np.testing.assert_allclose(fork[s], solo[0], rtol=0, atol=1e-14)
    # and a rollout's output does not move when another rollout's tokens do
    ak2 = ak.copy(); ak2[1] += 1.0
    fork2 = A.attention_step(q, shk, shv, [lp], ak2, av, blk_off, A.MASK_CAUSAL,
                             priv_k=pk, priv_v=pv, priv_len=priv)
    assert np.array_equal(fork[0], fork2[0]) and np.array_equal(fork[2], fork2[2])


def test_default_scale_is_inverse_sqrt_head_dim():
    R, Hq, Hkv, D, lp = 3, 2, 1, 16, 4
    q, pk, pv, ak, av = _one_seq(R, Hq, Hkv, D, lp, 12)
    a = A.attention_step(q, pk, pv, [lp], ak, av, [0, R], A.MASK_BIDIR)
    b = A.attention_step(q, pk, pv, [lp], ak, av, [0, R], A.MASK_BIDIR, scale=0.25)
    np.testing.assert_array_equal(a, b)
