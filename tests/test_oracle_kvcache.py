"""Pins of the KV-commit oracle: in-order append only, capacity bound."""

import numpy as np
import pytest

from oracle import kvcache as K


def test_commits_concatenate_in_order():
    rng = np.random.default_rng(0)
    pk = rng.standard_normal((2, 3, 8, 4)); pv = rng.standard_normal((2, 3, 8, 4))
    cache = K.new_cache(pk, pv, [2, 5])
    b1 = rng.standard_normal((3, 2, 4)); b2 = rng.standard_normal((3, 1, 4))
    assert K.commit(cache, 0, 2, b1, -b1) == 4
    assert K.commit(cache, 0, 4, b2, -b2) == 5
    k0, v0 = cache[0]
    assert np.array_equal(k0, np.concatenate([pk[0, :, :2], b1, b2], axis=1))
    assert np.array_equal(v0, np.concatenate([pv[0, :, :2], -b1, -b2], axis=1))
    assert np.array_equal(cache[1][0], pk[1, :, :5])          # other sequence untouched
    kp, vp = K.as_padded(cache, 8, np.float64)
    assert np.array_equal(kp[0, :, :5], k0) and not kp[0, :, 5:].any()


def test_out_of_order_and_capacity_rejected():
    pk = np.zeros((1, 1, 4, 2))
    cache = K.new_cache(pk, pk, [1])
    blk = np.ones((1, 2, 2))
    with pytest.raises(K.OrderError):
        K.commit(cache, 0, 0, blk, blk)
    with pytest.raises(K.OrderError):
        K.commit(cache, 0, 2, blk, blk)
    with pytest.raises(K.CapacityError):
        K.commit(cache, 0, 1, np.ones((1, 4, 2)), np.ones((1, 4, 2)), capacity=4)
    assert K.commit(cache, 0, 1, blk, blk, capacity=4) == 3
