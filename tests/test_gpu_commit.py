"""GPU parity of bc_kv_commit: the device cache equals the oracle's in-order
concatenation byte for byte; out-of-order and over-capacity commits are
rejected before any launch."""

import numpy as np
import pytest
import torch

from oracle import kvcache as OK
from tests import gpu_util as G
from block_causal_attention_gqa_amd import binding as B
from block_causal_attention_gqa_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    G.require_lib()


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64), ("bf16", 64)])
def test_section_commits_in_order(dtype, D):
    S, Hkv, cap = 2, 2, 3352
    lens0 = [3072, 3000]
    (k_t, v_t), (k32, v32) = synth.kv_cache(11, S, Hkv, cap, D, lens0, dtype)
    cache = B.KVCache(k_t.to(G.DEV), v_t.to(G.DEV))
    length = np.array(lens0, np.int32)
    ocache = OK.new_cache(k32, v32, lens0)
    for i, rows in enumerate([12, 32, 6, 32]):
        for s in range(S):
            bk = synth.normal(11, "commit_k", (Hkv, rows, D), i, s)
            bv = synth.normal(11, "commit_v", (Hkv, rows, D), i, s)
            bk_t, bk32 = synth.to_dtype(bk, dtype)
            bv_t, bv32 = synth.to_dtype(bv, dtype)
            B.bc_kv_commit(cache, length, s, int(length[s]), rows, bk_t.to(G.DEV), bv_t.to(G.DEV))
            OK.commit(ocache, s, int(length[s]) - rows, bk32, bv32, capacity=cap)
    torch.cuda.synchronize()
    kw, vw = OK.as_padded(ocache, cap, np.float32)
    assert list(length) == [3072 + 82, 3000 + 82]
    got_k = cache.k.float().cpu().numpy()
    got_v = cache.v.float().cpu().numpy()
    assert np.array_equal(got_k, kw) and np.array_equal(got_v, vw)


def test_order_and_capacity_errors():
    (k_t, v_t), _ = synth.kv_cache(12, 1, 2, 64, 128, [60], "bf16")
    cache = B.KVCache(k_t.to(G.DEV), v_t.to(G.DEV))
    length = np.array([60], np.int32)
    blk = torch.zeros((2, 4, 128), dtype=torch.bfloat16, device=G.DEV)
    assert B.bc_kv_commit(cache, length, 0, 59, 4, blk, blk, check=False) == B.BC_ERR_ORDER
    assert B.bc_kv_commit(cache, length, 0, 61, 1, blk, blk, check=False) == B.BC_ERR_ORDER
    big = torch.zeros((2, 5, 128), dtype=torch.bfloat16, device=G.DEV)
    assert B.bc_kv_commit(cache, length, 0, 60, 5, big, big, check=False) == B.BC_ERR_CAPACITY
    assert B.bc_kv_commit(cache, length, 1, 60, 1, blk, blk, check=False) == B.BC_ERR_ARG
    assert list(length) == [60]


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_commit_of_every_sequence_at_once(dtype, D):
    # seq = BC_ALL_SEQ: one launch commits [S][Hkv][rows][D] to all S
    # sequences, equal to S in-order single commits
    S, Hkv, cap = 5, 3, 300
    lens0 = [200] * S
    (k_t, v_t), (k32, v32) = synth.kv_cache(14, S, Hkv, cap, D, lens0, dtype)
    cache = B.KVCache(k_t.to(G.DEV), v_t.to(G.DEV))
    length = np.array(lens0, np.int32)
    ocache = OK.new_cache(k32, v32, lens0)
    for i, rows in enumerate([32, 1, 17]):
        bk = synth.normal(14, "commit_k", (S, Hkv, rows, D), i)
        bv = synth.normal(14, "commit_v", (S, Hkv, rows, D), i)
        bk_t, bk32 = synth.to_dtype(bk, dtype)
        bv_t, bv32 = synth.to_dtype(bv, dtype)
        B.bc_kv_commit(cache, length, B.BC_ALL_SEQ, int(length[0]), rows, bk_t.to(G.DEV), bv_t.to(G.DEV))
        for s in range(S):
            OK.commit(ocache, s, int(length[s]) - rows, bk32[s], bv32[s], capacity=cap)
    torch.cuda.synchronize()
    kw, vw = OK.as_padded(ocache, cap, np.float32)
    assert list(length) == [250] * S
    assert np.array_equal(cache.k.float().cpu().numpy(), kw) and np.array_equal(cache.v.float().cpu().numpy(), vw)
    # unequal lengths: the batched commit is out of order for someone
    length[2] += 1
    blk = torch.zeros((S, Hkv, 1, D), dtype=k_t.dtype, device=G.DEV)
    assert B.bc_kv_commit(cache, length, B.BC_ALL_SEQ, 250, 1, blk, blk, check=False) == B.BC_ERR_ORDER
