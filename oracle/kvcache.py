"""In-order KV commit -- oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

A block's K/V are cached once the block is complete, and only a completed
prefix whose predecessors are stable may be cached: commits are append-only
and in order (Fast-dVLA notes, key design 1; Fast-dDrive method summary
sec. 3.1 and "Section Diffusion").

The cache is a plain Python list with one entry per sequence; each entry is
a pair of arrays (K, V) shaped [Hkv][len][D], initially the prompt prefix.
"""

import numpy as np


class OrderError(ValueError):
    """A commit whose start row is not the sequence's current length."""


class CapacityError(ValueError):
    """A commit that would grow a sequence past the cache capacity."""


def new_cache(prefix_k, prefix_v, prefix_len):
    """Build the list-of-sequences cache from [S][Hkv][cap][D] arrays."""
    cache = []
    for s in range(len(prefix_len)):
        n = int(prefix_len[s])
        cache.append((np.array(prefix_k[s, :, :n]), np.array(prefix_v[s, :, :n])))
    return cache


def commit(cache, seq, start, blk_k, blk_v, capacity=None):
    """Append a completed block [Hkv][rows][D] to sequence ``seq``.

    ``start`` must equal the current length (else OrderError); the new length
    must not exceed ``capacity`` when one is given (else CapacityError).
    Returns the new length.
    """
    k, v = cache[seq]
    cur = k.shape[1]
    if start != cur:
        raise OrderError("commit at row %d but the sequence holds %d rows" % (start, cur))
    rows = blk_k.shape[1]
    if capacity is not None and cur + rows > capacity:
        raise CapacityError("commit of %d rows past capacity %d" % (rows, capacity))
    cache[seq] = (np.concatenate([k, blk_k], axis=1), np.concatenate([v, blk_v], axis=1))
    return cur + rows


def as_padded(cache, capacity, dtype):
    """The cache laid out as [S][Hkv][capacity][D] with zero rows past each
    sequence's length, for byte comparison with a device cache."""
    S = len(cache)
    Hkv, _, D = cache[0][0].shape
    k_out = np.zeros((S, Hkv, capacity, D), dtype=dtype)
    v_out = np.zeros((S, Hkv, capacity, D), dtype=dtype)
    for s, (k, v) in enumerate(cache):
        k_out[s, :, :k.shape[1]] = k
        v_out[s, :, :v.shape[1]] = v
    return k_out, v_out
