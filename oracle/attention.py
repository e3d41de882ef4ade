"""Block-causal GQA attention over a committed KV prefix -- float64 oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What is computed (restated from the pages, not copied):
  * The output of a block-diffusion decoder is cut into blocks.  Inside a
    block attention is bidirectional; across blocks it is causal, so a block
    sees the prompt prefix, every earlier block and itself, never a later
    block (WAM-Diff2 article sec. 2.1; Fast-dVLA notes, key design 1;
    Fast-dDrive method summary sec. 3.1).
  * Completed blocks never change again, so their K/V are read from a cache
    instead of being recomputed (Fast-dDrive sec. 1; Fast-dVLA notes, key
    design 1; method summary sec. 3.1).
  * The AR verify pass of scaffold speculative decoding runs one causal pass
    over the block: row i sees only positions before and at i (method summary
    sec. 3.2, "Scaffold Speculative Decoding", step 3).
  * N rollouts fork from one shared prefix KV cache: a rollout sees the shared
    prefix, its own private blocks and its own active block, never another
    rollout's tokens (Fast-dDrive abstract; method summary sec. 3.3).

Readings where the pages are silent: the softmax scale is an explicit
argument (1/sqrt(head_dim) by default); query head h reads KV head
h // (n_q_heads / n_kv_heads); every prefix key is visible to every active
query.

Layouts (NumPy arrays, any float dtype; promoted to float64):
  q          [S][R][Hq][D]        active query rows
  prefix_k/v [Sp][Hkv][cap][D]    committed cache; Sp == S, or Sp == 1 (fork)
  prefix_len [Sp]                 valid rows of each prefix cache
  priv_k/v   [S][Hkv][capv][D]    fork only: each rollout's private cache
  priv_len   [S]
  active_k/v [S][Hkv][R][D]       the active rows' own K/V (recomputed per step)
  blk_off    [n_blk + 1]          active block boundaries, 0 .. R, increasing
"""

import numpy as np

MASK_BIDIR = 0   # bidirectional inside a block, causal across blocks
MASK_CAUSAL = 1  # causal inside a block too (the AR verify pass)


def block_of_rows(blk_off):
    """Block index of every active row: row j is in block b when
    blk_off[b] <= j < blk_off[b + 1]."""
    blk_off = np.asarray(blk_off, dtype=np.int64)
    n_rows = int(blk_off[-1])
    blk = np.empty(n_rows, dtype=np.int64)
    for b in range(len(blk_off) - 1):
        blk[blk_off[b]:blk_off[b + 1]] = b
    return blk


def active_visibility(blk_off, mode):
    """Boolean [R][R] matrix: entry [i, j] says whether active query row i may
    read active key row j.

    BIDIR:  block(j) <= block(i).
    CAUSAL: block(j) <  block(i), or the same block and j <= i.
    """
    blk = block_of_rows(blk_off)
    bi = blk[:, None]
    bj = blk[None, :]
    if mode == MASK_BIDIR:
        return bj <= bi
    if mode == MASK_CAUSAL:
        i = np.arange(len(blk))[:, None]
        j = np.arange(len(blk))[None, :]
        return (bj < bi) | ((bj == bi) & (j <= i))
    raise ValueError("unknown mask mode %r" % (mode,))


def masked_softmax_attention(q, k, v, visible, scale):
    """One head: q [R][D], k/v [L][D], visible [R][L] -> out [R][D].

    s = scale * q k^T; hidden entries are set to -inf; p = softmax(s) over the
    key axis; out = p v.  Every row must see at least one key.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = scale * (q @ k.T)
    s = np.where(visible, s, -np.inf)
    s_max = s.max(axis=1, keepdims=True)
    if not np.all(np.isfinite(s_max)):
        raise ValueError("a query row sees no key")
    p = np.exp(s - s_max)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ v


def attention_step(q, prefix_k, prefix_v, prefix_len, active_k, active_v,
                   blk_off, mode, scale=None,
                   priv_k=None, priv_v=None, priv_len=None):
    """Attention of every active query row of every sequence / rollout.

    Returns float64 [S][R][Hq][D].  With ``priv_k`` given this is the
    shared-prefix fork: prefix_* hold one sequence that all S rollouts read.
    """
    q = np.asarray(q)
    S, R, Hq, D = q.shape
    Sp, Hkv = prefix_k.shape[0], prefix_k.shape[1]
    fork = priv_k is not None
    if fork and Sp != 1:
        raise ValueError("fork: the shared prefix holds exactly one sequence")
    if not fork and Sp != S:
        raise ValueError("one prefix cache per sequence")
    if Hq % Hkv:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    if int(np.asarray(blk_off)[-1]) != R:
        raise ValueError("blk_off must end at n_rows")
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    act_vis = active_visibility(blk_off, mode)

    out = np.zeros((S, R, Hq, D), dtype=np.float64)
    for s in range(S):
        ps = 0 if fork else s
        lp = int(prefix_len[ps])
        parts_k = [prefix_k[ps, :, :lp]]
        parts_v = [prefix_v[ps, :, :lp]]
        n_always = lp
        if fork:
            lv = int(priv_len[s])
            parts_k.append(priv_k[s, :, :lv])
            parts_v.append(priv_v[s, :, :lv])
            n_always += lv
        parts_k.append(active_k[s])
        parts_v.append(active_v[s])
        keys = np.concatenate([np.asarray(x, dtype=np.float64) for x in parts_k], axis=1)
        vals = np.concatenate([np.asarray(x, dtype=np.float64) for x in parts_v], axis=1)
        visible = np.concatenate(
            [np.ones((R, n_always), dtype=bool), act_vis], axis=1)
        for h in range(Hq):
            kv = h // group
            out[s, :, h, :] = masked_softmax_attention(
                q[s, :, h, :], keys[kv], vals[kv], visible, scale)
    return out


def full_sequence_attention(q, k, v, blk, mode, scale=None):
    """Full recompute over one whole sequence under the block-causal mask.

    q [N][Hq][D], k/v [N][Hkv][D], blk [N] = non-decreasing block id of every
    position (the prompt prefix is simply the lowest block id(s)).  Position i
    reads position j when blk[j] < blk[i], or blk[j] == blk[i] and (BIDIR, or
    j <= i under CAUSAL).  Returns float64 [N][Hq][D].

    This is the formulation without a KV cache: every position is recomputed
    from scratch, so the cached-prefix path can be checked against it.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    blk = np.asarray(blk)
    N, Hq, D = q.shape
    Hkv = k.shape[1]
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    bi = blk[:, None]
    bj = blk[None, :]
    if mode == MASK_BIDIR:
        visible = bj <= bi
    else:
        i = np.arange(N)[:, None]
        j = np.arange(N)[None, :]
        visible = (bj < bi) | ((bj == bi) & (j <= i))
    out = np.zeros((N, Hq, D), dtype=np.float64)
    for h in range(Hq):
        out[:, h, :] = masked_softmax_attention(
            q[:, h, :], k[:, h // group, :], v[:, h // group, :], visible, scale)
    return out

