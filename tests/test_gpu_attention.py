"""GPU parity of bc_attn_step against the float64 oracle.

Tolerances: max-abs 1e-5 for float32 inputs, 1e-2 for bf16 inputs (float32
accumulation, bf16 probabilities into the PV product, bf16 output)."""

import numpy as np
import pytest

from oracle import attention as OA
from tests import gpu_util as G
from block_causal_attention_gqa_amd import binding as B

pytestmark = pytest.mark.gpu

BIDIR, CAUSAL = B.BC_MASK_BLOCK_BIDIR, B.BC_MASK_BLOCK_CAUSAL
TOL = {"f32": 1e-5, "bf16": 1e-2}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    G.require_lib()


def _check(seed, S, R, Hq, Hkv, D, dtype, prefix_len, blk_off, mode, **kw):
    print("attn case seed=%d S=%d R=%d Hq=%d Hkv=%d D=%d %s prefix=%s blk=%s mode=%d %s"
          % (seed, S, R, Hq, Hkv, D, dtype, list(prefix_len)[:4], list(blk_off)[:6], mode, kw), flush=True)
    got, h = G.attn_case(seed, S, R, Hq, Hkv, D, dtype, prefix_len, blk_off, mode, **kw)
    fork = kw.get("fork", False)
    want = OA.attention_step(h["q"], h["pk"], h["pv"], prefix_len, h["k"], h["v"], blk_off, mode,
                             scale=h["scale"], priv_k=h["vk"] if fork else None,
                             priv_v=h["vv"] if fork else None,
                             priv_len=kw.get("priv_len") if fork else None)
    err = np.abs(got - want).max()
    assert err <= TOL[dtype], "max-abs %.3g > %.3g" % (err, TOL[dtype])
    return got


def test_tiny_fp32_single_step():
    # 1 sequence, 4 query heads / 1 KV head, head_dim 64, fp32, prefix 256 + one block of 8
    _check(0, 1, 8, 4, 1, 64, "f32", [256], [0, 8], BIDIR)


@pytest.mark.parametrize("splits", [0, 1, 3, 7, 40])
def test_tiny_fp32_split_counts(splits):
    _check(1, 1, 8, 4, 1, 64, "f32", [256], [0, 8], BIDIR, n_splits=splits)


@pytest.mark.parametrize("bs", [32, 12, 6])
def test_section_decode_shape(bs):
    # Fast-dDrive section decode: bs1, 16q/2kv, D 128, bf16, prefix 3072 + a block
    _check(2, 1, bs, 16, 2, 128, "bf16", [3072], [0, bs], BIDIR, cap=3352)


def test_section_decode_grown_prefix():
    _check(3, 1, 32, 16, 2, 128, "bf16", [3072 + 236], [0, 32], BIDIR, cap=3352)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
@pytest.mark.parametrize("mode", [BIDIR, CAUSAL])
def test_ragged_multiblock(D, group, mode):
    Hkv = 2
    _check(10 + group, 1, 23, Hkv * group, Hkv, D, "bf16", [333], [0, 5, 17, 23], mode, cap=400)


@pytest.mark.parametrize("splits", [1, 2, 5, 64])
def test_forced_splits_with_empty_chunks(splits):
    _check(20, 1, 17, 8, 2, 128, "bf16", [97], [0, 9, 17], CAUSAL, cap=200, n_splits=splits)


def test_empty_prefix():
    _check(21, 1, 9, 4, 2, 128, "bf16", [0], [0, 4, 9], BIDIR, cap=64)


def test_fp32_multiblock_causal():
    _check(22, 2, 13, 6, 3, 128, "f32", [70, 141], [0, 7, 13], CAUSAL, cap=160)


def test_large_block_batch_independent_prefixes():
    # WAM-Diff2 shape: 32q/8kv, D 128, bf16, prefix 2048, block of 32, batch 4
    _check(30, 4, 32, 32, 8, 128, "bf16", [2048, 2080, 2112, 2304], [0, 32], BIDIR, cap=2304)


def test_pipelined_three_active_blocks():
    # Fast-dVLA: 3 active 7-token blocks over a 512-token prefix
    _check(40, 1, 21, 16, 2, 128, "bf16", [512], [0, 7, 14, 21], BIDIR)


def test_pipelined_625_window():
    # 625-token output in blocks of 32, window of 3 active blocks (96 rows)
    _check(41, 1, 96, 16, 2, 128, "bf16", [512 + 32 * 9], [0, 32, 64, 96], BIDIR, cap=1137)
    _check(42, 1, 81, 16, 2, 128, "bf16", [512 + 32 * 17], [0, 32, 64, 81], BIDIR, cap=1137)


@pytest.mark.parametrize("mode", [BIDIR, CAUSAL])
@pytest.mark.parametrize("N", [1, 4])
def test_fork_shared_prefix(mode, N):
    # shared prefix 3072 + 210, 16q/2kv, trajectory block of 24 rows, private
    # blocks of earlier trajectory blocks per rollout
    priv = [0, 24, 47, 23][:N]
    _check(50 + N, N, 24, 16, 2, 128, "bf16", [3282], [0, 24], mode, fork=True,
           priv_len=priv, priv_cap=48)


def test_fork_sixteen_rollouts_ragged_rows():
    priv = [(7 * s) % 48 for s in range(16)]
    _check(60, 16, 23, 16, 2, 128, "bf16", [3282], [0, 23], CAUSAL, fork=True, priv_len=priv, priv_cap=48)


# ---- many rows per KV-head group (>= 2048 rows): 128-row tiles with two
# 16-row column tiles per wave, long items


@pytest.mark.parametrize("mode", [BIDIR, CAUSAL])
def test_fork_sixtyfour_rollouts(mode):
    # the fork at full size: 64 rollouts x 24 rows x 8 heads per KV head
    priv = [(11 * s) % 48 for s in range(64)]
    _check(64, 64, 24, 16, 2, 128, "bf16", [3282], [0, 24], mode, fork=True, priv_len=priv, priv_cap=48)


@pytest.mark.parametrize("splits", [0, 1, 3])
@pytest.mark.parametrize("mode", [BIDIR, CAUSAL])
def test_many_rows_head_dim_64(mode, splits):
    # 512 rows x group 4: 2048 rows per group, ragged prefix, uneven blocks
    _check(70 + splits, 1, 512, 16, 4, 64, "bf16", [1000], [0, 100, 256, 300, 512], mode, n_splits=splits)


def test_many_rows_empty_prefix():
    # no committed keys: the prefix items have no tiles, the active items do all the work
    _check(75, 1, 1024, 4, 1, 128, "bf16", [0], [0, 512, 1024], CAUSAL)


# ---- many sequences, each with its own prefix of very different length


@pytest.mark.parametrize("splits", [0, 2, 3])
@pytest.mark.parametrize("mode", [BIDIR, CAUSAL])
def test_batch_ragged_prefixes(mode, splits):
    # 8 sequences x 4 KV heads: 32 groups of 32 rows x 4 heads (128 rows);
    # prefixes from empty to 2047 keys, so a call's items run from 0 to 16
    # key tiles; blocks of 7 / 13 / 12
    lens = [2047, 64, 0, 300, 517, 1000, 1999, 130]
    _check(80 + splits, 8, 32, 16, 4, 128, "bf16", lens, [0, 7, 20, 32], mode, cap=2048, n_splits=splits)


@pytest.mark.parametrize("mode", [BIDIR, CAUSAL])
def test_batch16_ragged_prefixes_with_short_ones(mode):
    # 16 sequences x 8 KV heads of 2 query heads: 128 row tiles of 64 rows
    # (32 rows x 2 heads); prefixes from empty to 2047 keys, several shorter
    # than one key tile or one split
    lens = [0, 5, 64, 100, 130, 300, 2047, 1999, 1500, 1024, 777, 65, 2000, 1234, 640, 191]
    _check(86, 16, 32, 16, 8, 128, "bf16", lens, [0, 7, 20, 32], mode, cap=2048)


def test_batch16_ragged_prefixes_folded():
    # the large-block batch-16 shape (32q/8kv, 32-row block) with ragged
    # prefixes: 512 prefix items, the active keys folded into the last chunk
    lens = [2176 - 37 * s for s in range(16)]
    _check(85, 16, 32, 32, 8, 128, "bf16", lens, [0, 32], BIDIR, cap=2176)


def test_block_size_one_equals_causal():
    # WAM-Diff2 sec. 2.1: B = 1 is causal decoding -- bitwise equal on the GPU
    a, _ = G.attn_case(70, 1, 16, 8, 2, 128, "bf16", [300], list(range(17)), BIDIR)
    b, _ = G.attn_case(70, 1, 16, 8, 2, 128, "bf16", [300], [0, 16], CAUSAL)
    assert np.array_equal(a, b)


def test_completed_block_rows_do_not_move():
    # rows of earlier blocks are bit-identical when a later block's inputs
    # change (Fast-dVLA notes, key design 1)
    import torch
    from block_causal_attention_gqa_amd import synth
    seed, R, Hq, Hkv, D = 71, 20, 8, 2, 128
    (pk_t, pv_t), _ = synth.kv_cache(seed, 1, Hkv, 256, D, [256], "bf16")
    (q_t, _), (k_t, _), (v_t, _) = synth.active_qkv(seed, 1, R, Hq, Hkv, D, "bf16", 0)
    prefix = B.KVCache(pk_t.to(G.DEV), pv_t.to(G.DEV))
    blk = [0, 8, 20]
    nb = B.bc_attn_workspace_bytes(prefix, None, (1, R, Hq, D), blk)
    ws = torch.empty(nb, dtype=torch.uint8, device=G.DEV)
    outs = []
    for variant in range(2):
        q, k, v = q_t.clone(), k_t.clone(), v_t.clone()
        if variant:
            q[0, 8:] = -q[0, 8:]
            k[0, :, 8:] = k[0, :, 8:] * 2
            v[0, :, 8:] = v[0, :, 8:] + 1
        out = torch.empty((1, R, Hq, D), dtype=torch.bfloat16, device=G.DEV)
        B.bc_attn_step(prefix, [256], None, None, q.to(G.DEV), k.to(G.DEV), v.to(G.DEV), blk, BIDIR,
                       D ** -0.5, out, ws)
        outs.append(out.cpu())
    assert torch.equal(outs[0][0, :8], outs[1][0, :8])
    assert not torch.equal(outs[0][0, 8:], outs[1][0, 8:])


def test_workspace_and_argument_errors_before_launch():
    import torch
    from block_causal_attention_gqa_amd import synth
    (pk_t, pv_t), _ = synth.kv_cache(1, 1, 2, 128, 128, [100], "bf16")
    (q_t, _), (k_t, _), (v_t, _) = synth.active_qkv(1, 1, 8, 16, 2, 128, "bf16", 0)
    prefix = B.KVCache(pk_t.to(G.DEV), pv_t.to(G.DEV))
    out = torch.empty((1, 8, 16, 128), dtype=torch.bfloat16, device=G.DEV)
    nb = B.bc_attn_workspace_bytes(prefix, None, (1, 8, 16, 128), [0, 8])
    q, k, v = q_t.to(G.DEV), k_t.to(G.DEV), v_t.to(G.DEV)
    # too small for a single split
    tiny = torch.empty(256, dtype=torch.uint8, device=G.DEV)
    st = B.bc_attn_step(prefix, [100], None, None, q, k, v, [0, 8], BIDIR, 0.1, out, tiny, check=False)
    assert st == B.BC_ERR_WORKSPACE
    # an explicit split count must fit the workspace
    nb3 = B.bc_attn_workspace_bytes(prefix, None, (1, 8, 16, 128), [0, 8], 3)
    small = torch.empty(nb3 - 256, dtype=torch.uint8, device=G.DEV)
    st = B.bc_attn_step(prefix, [100], None, None, q, k, v, [0, 8], BIDIR, 0.1, out, small, n_prefix_splits=3,
                        check=False)
    assert st == B.BC_ERR_WORKSPACE
    ws = torch.empty(nb, dtype=torch.uint8, device=G.DEV)
    assert B.bc_attn_step(prefix, [129], None, None, q, k, v, [0, 8], BIDIR, 0.1, out, ws,
                          check=False) == B.BC_ERR_ARG
    assert B.bc_attn_step(prefix, [100], None, None, q, k, v, [0, 5, 5, 8], BIDIR, 0.1, out, ws,
                          check=False) == B.BC_ERR_ARG
    assert B.bc_attn_step(prefix, [100], None, None, q, k, v, [0, 8], 7, 0.1, out, ws,
                          check=False) == B.BC_ERR_ARG


def test_partial_then_combine_equals_step():
    import torch
    from block_causal_attention_gqa_amd import synth
    seed, S, R, Hq, Hkv, D = 80, 2, 19, 16, 2, 128
    (pk, pv), _ = synth.kv_cache(seed, S, Hkv, 700, D, [650, 333], "bf16")
    (q, _), (k, _), (v, _) = synth.active_qkv(seed, S, R, Hq, Hkv, D, "bf16", 0)
    prefix = B.KVCache(pk.to(G.DEV), pv.to(G.DEV))
    q, k, v = q.to(G.DEV), k.to(G.DEV), v.to(G.DEV)
    ws = torch.empty(B.bc_attn_workspace_bytes(prefix, None, (S, R, Hq, D), [0, 7, 19]), dtype=torch.uint8,
                     device=G.DEV)
    a = torch.empty((S, R, Hq, D), dtype=torch.bfloat16, device=G.DEV)
    b = torch.empty_like(a)
    args = (prefix, [650, 333], None, None, q, k, v, [0, 7, 19], CAUSAL, D ** -0.5)
    B.bc_attn_step(*args, a, ws)
    B.bc_attn_partial(*args, b, ws)
    B.bc_attn_combine(*args, b, ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ---- the fork at N >= 64 rollouts: one workgroup per half of a rollout's
# rows over all their keys (shared prefix, private keys, active keys), in two
# key halves merged in LDS, the output written without a combine


@pytest.mark.parametrize("mode", [BIDIR, CAUSAL])
@pytest.mark.parametrize("prefix", [0, 70, 1000])
def test_fork_sixtyfour_short_prefixes_odd_rows(mode, prefix):
    # 23-row blocks (184 rows per rollout and KV head: half tiles of 92),
    # shared prefixes from empty to 1000 keys, private lengths 0 .. 47, two
    # blocks inside the active rows
    priv = [(13 * s) % 48 for s in range(64)]
    _check(95, 64, 23, 16, 2, 128, "bf16", [prefix], [0, 9, 23], mode, fork=True, priv_len=priv, priv_cap=48,
           cap=max(prefix, 1))


@pytest.mark.parametrize("N,mode", [(16, BIDIR), (32, CAUSAL)])
def test_fork_row_tiles_with_key_splits(N, mode):
    # N = 16 / 32 rollouts over the full 3282-key prefix: 4 / 2 key splits
    # per row tile (one workgroup per CU), split records merged by the
    # combine; two blocks inside the active rows, private lengths 0 .. 47
    priv = [(7 * s + 3) % 48 for s in range(N)]
    _check(98 + N, N, 24, 16, 2, 128, "bf16", [3282], [0, 10, 24], mode, fork=True, priv_len=priv, priv_cap=48)


@pytest.mark.parametrize("N", [16, 64])
def test_fork_row_tiles_partial_then_combine_equals_step(N):
    # N = 64: the partial pass writes the output itself and the combine does
    # nothing; N = 16: split records, merged by the combine
    import torch
    from block_causal_attention_gqa_amd import synth
    seed, R, Hq, Hkv, D = 96, 24, 16, 2, 128
    (pk, pv), _ = synth.kv_cache(seed, 1, Hkv, 3282, D, [3282], "bf16")
    priv_len = [(5 * s) % 48 for s in range(N)]
    (vk, vv), _ = synth.kv_cache(seed, N, Hkv, 48, D, priv_len, "bf16", purpose=("priv_k", "priv_v"))
    (q, _), (k, _), (v, _) = synth.active_qkv(seed, N, R, Hq, Hkv, D, "bf16", 0)
    prefix, priv = B.KVCache(pk.to(G.DEV), pv.to(G.DEV)), B.KVCache(vk.to(G.DEV), vv.to(G.DEV))
    q, k, v = q.to(G.DEV), k.to(G.DEV), v.to(G.DEV)
    ws = torch.empty(B.bc_attn_workspace_bytes(prefix, priv, (N, R, Hq, D), [0, R]), dtype=torch.uint8,
                     device=G.DEV)
    a = torch.empty((N, R, Hq, D), dtype=torch.bfloat16, device=G.DEV)
    b = torch.full_like(a, 7.0)
    args = (prefix, [3282], priv, priv_len, q, k, v, [0, R], BIDIR, D ** -0.5)
    B.bc_attn_step(*args, a, ws)
    B.bc_attn_partial(*args, b, ws)
    B.bc_attn_combine(*args, b, ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_fork_sixtyfour_forced_splits_agree_with_direct_form():
    # an explicit split count takes the split plan (partials and combine);
    # both forms match the oracle and each other within the bf16 tolerance
    priv = [(11 * s) % 48 for s in range(64)]
    d = _check(97, 64, 24, 16, 2, 128, "bf16", [3282], [0, 24], CAUSAL, fork=True, priv_len=priv, priv_cap=48)
    f = _check(97, 64, 24, 16, 2, 128, "bf16", [3282], [0, 24], CAUSAL, fork=True, priv_len=priv, priv_cap=48,
               n_splits=2)
    assert np.abs(d - f).max() <= 2 * TOL["bf16"]


def test_automatic_splits_shrink_to_the_workspace():
    # a workspace that holds fewer slots than the automatic choice wants:
    # the call uses fewer splits and the result still matches the oracle
    import torch
    from block_causal_attention_gqa_amd import synth
    seed, S, R, Hq, Hkv, D = 90, 1, 32, 16, 2, 128
    (pk, pv), (k32, v32) = synth.kv_cache(seed, S, Hkv, 3352, D, [3100], "bf16")
    (q, q32), (k, ka), (v, va) = synth.active_qkv(seed, S, R, Hq, Hkv, D, "bf16", 0)
    prefix = B.KVCache(pk.to(G.DEV), pv.to(G.DEV))
    full = B.bc_attn_workspace_bytes(prefix, None, (S, R, Hq, D), [0, R])
    one = B.bc_attn_workspace_bytes(prefix, None, (S, R, Hq, D), [0, R], 1)
    assert one < full
    out = torch.empty((S, R, Hq, D), dtype=torch.bfloat16, device=G.DEV)
    want = OA.attention_step(q32, k32, v32, [3100], ka, va, [0, R], BIDIR, scale=D ** -0.5)
    for nbytes in (one, (one + full) // 2, full):
        ws = torch.empty(nbytes, dtype=torch.uint8, device=G.DEV)
        B.bc_attn_step(prefix, [3100], None, None, q.to(G.DEV), k.to(G.DEV), v.to(G.DEV), [0, R], BIDIR,
                       D ** -0.5, out, ws)
        got = out.float().cpu().numpy()
        assert np.abs(got - want).max() <= TOL["bf16"]


# ---- fold: without a fork, when the prefix items fill the co-resident
# workgroups but the active items would not fit beside them, the last prefix
# chunk of each row tile also takes its active keys.  16 sequences x 8 KV
# heads x 32 rows x 4 query heads: 256 row tiles of 64 rows, so two chunks
# give 512 prefix items and 256 active items (folded); one chunk gives 256 +
# 256 (resident together) and three give 768 prefix items (more than one
# round anyway): both keep the active items apart.  The lengths put the last
# chunk's prefix keys at zero (the active keys become the item's only
# segment), at partial tiles, and at whole tiles.


@pytest.mark.parametrize("splits", [1, 2, 3])
@pytest.mark.parametrize("mode", [BIDIR, CAUSAL])
def test_fold_active_keys_into_the_last_chunk(mode, splits):
    lens = [0, 1, 40, 63, 64, 65, 127, 300, 511, 512, 700, 1000, 1023, 1024, 1100, 1200]
    _check(120 + splits, 16, 32, 32, 8, 128, "bf16", lens, [0, 7, 19, 32], mode, cap=1200, n_splits=splits)


def test_fold_head_dim_64_automatic_splits():
    lens = [int(x) for x in np.random.default_rng(124).integers(0, 2049, 16)]
    _check(124, 16, 32, 32, 8, 64, "bf16", lens, [0, 32], BIDIR, cap=2048, n_splits=2)
    _check(125, 16, 32, 32, 8, 64, "bf16", lens, [0, 32], BIDIR, cap=2048)


# ---- the call limits: BC_MAX_BLOCKS active blocks, BC_MAX_SEQ sequences


@pytest.mark.parametrize("mode", [BIDIR, CAUSAL])
def test_max_blocks_ragged(mode):
    # 64 active blocks of 1..9 rows over two ragged prefixes
    sizes = np.random.default_rng(100).integers(1, 10, B.BC_MAX_BLOCKS)
    off = np.concatenate([[0], np.cumsum(sizes)]).tolist()
    _check(100 + mode, 2, off[-1], 16, 2, 128, "bf16", [700, 123], off, mode, cap=700)


def test_max_sequences_own_prefixes():
    # 64 sequences, each with its own prefix length (some empty, some one key)
    lens = [0, 1, 900] + np.random.default_rng(101).integers(0, 901, B.BC_MAX_SEQ - 3).tolist()
    _check(101, B.BC_MAX_SEQ, 12, 8, 2, 64, "bf16", lens, [0, 5, 12], BIDIR, cap=900)


def test_max_sequences_and_max_blocks():
    # 64 sequences x 64 blocks of one row: block-bidirectional with blocks of
    # size one is causal decoding, and both masks give the oracle's result
    lens = np.random.default_rng(102).integers(0, 301, B.BC_MAX_SEQ).tolist()
    off = list(range(B.BC_MAX_BLOCKS + 1))
    a = _check(102, B.BC_MAX_SEQ, B.BC_MAX_BLOCKS, 4, 1, 64, "bf16", lens, off, BIDIR, cap=300)
    b = _check(102, B.BC_MAX_SEQ, B.BC_MAX_BLOCKS, 4, 1, 64, "bf16", lens, [0, B.BC_MAX_BLOCKS], CAUSAL,
               cap=300)
    assert np.array_equal(a, b)


def test_one_past_the_sequence_and_block_limits_is_unsupported():
    import torch
    from block_causal_attention_gqa_amd import synth
    D, Hq, Hkv = 64, 4, 1
    for S, R, off in [(B.BC_MAX_SEQ + 1, 2, [0, 2]),
                      (1, B.BC_MAX_BLOCKS + 1, list(range(B.BC_MAX_BLOCKS + 2)))]:
        (pk, pv), _ = synth.kv_cache(103, S, Hkv, 16, D, [16] * S, "bf16")
        (q, _), (k, _), (v, _) = synth.active_qkv(103, S, R, Hq, Hkv, D, "bf16", 0)
        prefix = B.KVCache(pk.to(G.DEV), pv.to(G.DEV))
        out = torch.empty((S, R, Hq, D), dtype=torch.bfloat16, device=G.DEV)
        ws = torch.empty(1 << 20, dtype=torch.uint8, device=G.DEV)
        assert B.bc_attn_workspace_bytes(prefix, None, (S, R, Hq, D), off) == 0
        st = B.bc_attn_step(prefix, [16] * S, None, None, q.to(G.DEV), k.to(G.DEV), v.to(G.DEV), off, BIDIR,
                            0.125, out, ws, check=False)
        assert st == B.BC_ERR_UNSUPPORTED


# ---- split partial formats: float32 below 1024 output rows, compact (int16
# against a power of two per row and slot) from 1024 rows with bf16 inputs


@pytest.mark.parametrize("splits", [1, 5, 64])
def test_compact_partials_with_empty_chunks(splits):
    # 128 rows x 8 heads = 1024 output rows; most of the forced chunks of a
    # 97-key prefix are empty
    _check(111, 1, 128, 8, 2, 128, "bf16", [97], [0, 40, 128], CAUSAL, cap=200, n_splits=splits)


@pytest.mark.parametrize("R", [32, 128])   # 512 output rows: float32 partials; 2048: compact
def test_output_scales_exactly_with_power_of_two_values(R):
    # Scaling V by a power of two scales every partial, every record's scale
    # and the merged output by the same power of two, with no new rounding:
    # the outputs must match bit for bit, and V = 0 must give exactly 0.
    import torch
    from block_causal_attention_gqa_amd import synth
    seed, S, Hq, Hkv, D, L = 112, 1, 16, 2, 128, 1500
    (pk, pv), _ = synth.kv_cache(seed, S, Hkv, L, D, [L], "bf16")
    (q, _), (k, _), (v, _) = synth.active_qkv(seed, S, R, Hq, Hkv, D, "bf16", 0)
    blk = [0, R // 2, R]
    ws = torch.zeros(B.bc_attn_workspace_bytes(B.KVCache(pk.to(G.DEV), pv.to(G.DEV)), None, (S, R, Hq, D), blk),
                     dtype=torch.uint8, device=G.DEV)
    outs = {}
    for f in (1.0, 2.0 ** 10, 2.0 ** -20, 0.0):
        prefix = B.KVCache(pk.to(G.DEV), (pv * f).to(G.DEV))
        out = torch.empty((S, R, Hq, D), dtype=torch.bfloat16, device=G.DEV)
        B.bc_attn_step(prefix, [L], None, None, q.to(G.DEV), k.to(G.DEV), (v * f).to(G.DEV), blk, BIDIR,
                       D ** -0.5, out, ws)
        torch.cuda.synchronize()
        outs[f] = out.float().cpu()
    assert outs[1.0].abs().max() > 0.1
    assert torch.equal(outs[2.0 ** 10], outs[1.0] * 2.0 ** 10)
    assert torch.equal(outs[2.0 ** -20], outs[1.0] * 2.0 ** -20)
    assert not outs[0.0].any()


def test_fp32_many_rows_keeps_float32_partials():
    # 2 x 64 rows x 8 heads = 1024 output rows: bf16 inputs would take the
    # compact partials here; float32 inputs keep float32 ones and the 1e-5 bound
    _check(113, 2, 64, 8, 2, 64, "f32", [500, 257], [0, 30, 64], CAUSAL, cap=500)


@pytest.mark.parametrize("mode", [BIDIR, CAUSAL])
def test_fork_head_dim_64(mode):
    # compact partials and the 8-value combine at head_dim 64: 16 rollouts x
    # 24 rows x 8 heads per KV head
    priv = [(13 * s) % 48 for s in range(16)]
    _check(114, 16, 24, 16, 2, 64, "bf16", [1500], [0, 24], mode, fork=True, priv_len=priv, priv_cap=48)


# ---- a running maximum that jumps: the online softmax's rescale.  With N(0,1)
# inputs a row's scaled scores stay within a few units, so after the first key
# tile no tile raises the running maximum by more than the rescale slack (8 in
# log2 units, 8 ln 2 = 5.5 in natural units) and the rescale of a non-empty
# accumulator never runs.  Here chosen key ranges get raised scores
# (G.biased_keys), so that a row's maximum climbs by 8-20 units several times:
# inside a chunk, across split chunks (the combine), across the fork's key
# halves (the merge in LDS), and between prefix, private and active keys.

SLACK_NAT = 8 * np.log(2.0)


def _steps(levels, width):
    lv = np.asarray(levels, np.float64)
    return lambda j: lv[np.minimum(np.asarray(j) // width, len(lv) - 1)]


def _const(c):
    return lambda j: np.full(len(j), float(c))


PREFIX_JUMPS = _steps([0, 4, 12, 20, 8, 16], 512)


def _check_biased(seed, S, R, Hq, Hkv, D, dtype, prefix_len, blk_off, mode, bias, **kw):
    print("attn biased case seed=%d S=%d R=%d Hq=%d Hkv=%d D=%d %s prefix=%s blk=%s mode=%d %s"
          % (seed, S, R, Hq, Hkv, D, dtype, list(prefix_len)[:4], list(blk_off)[:6], mode, kw), flush=True)
    got, h = G.attn_case(seed, S, R, Hq, Hkv, D, dtype, prefix_len, blk_off, mode, key_bias=bias, **kw)
    fork = kw.get("fork", False)
    want = OA.attention_step(h["q"], h["pk"], h["pv"], prefix_len, h["k"], h["v"], blk_off, mode,
                             scale=h["scale"], priv_k=h["vk"] if fork else None,
                             priv_v=h["vv"] if fork else None,
                             priv_len=kw.get("priv_len") if fork else None)
    err = np.abs(got - want).max()
    assert err <= TOL[dtype], "max-abs %.3g > %.3g" % (err, TOL[dtype])
    # the inputs do what they are for: over the first sequence's prefix, the
    # first row's running maximum (moved only past the slack, as the kernels
    # move theirs) is raised by a 64-key tile at least twice
    sc = h["pk"][0, 0, :prefix_len[0]].astype(np.float64) @ h["q"][0, 0, 0].astype(np.float64) * h["scale"]
    tiles = [sc[i:i + 64].max() for i in range(0, len(sc), 64)]
    m, moves = tiles[0], 0
    for t in tiles[1:]:
        if t > m + SLACK_NAT:
            m, moves = t, moves + 1
    assert moves >= 2, "the running maximum moved %d times" % moves


@pytest.mark.parametrize("splits", [0, 1, 4])
@pytest.mark.parametrize("mode", [BIDIR, CAUSAL])
def test_running_max_jumps_section_shape(mode, splits):
    # bs1 section shape; splits 0: the automatic split (about 25 chunks of two
    # tiles, float32 records); 1: one chunk over the whole prefix
    bias = dict(prefix=PREFIX_JUMPS, active=_const(22.0))
    _check_biased(90 + splits, 1, 32, 16, 2, 128, "bf16", [3072], [0, 12, 32], mode, bias, cap=3352,
                  n_splits=splits)


def test_running_max_jumps_many_rows_head_dim_64():
    # 2048 rows per group: 128-row tiles of two column tiles, compact records
    bias = dict(prefix=_steps([0, 9, 18], 320), active=lambda j: 14.0 + 0.02 * np.asarray(j))
    _check_biased(98, 1, 512, 16, 4, 64, "bf16", [1000], [0, 100, 256, 300, 512], CAUSAL, bias)


def test_running_max_jumps_batch16_folded():
    # the large-block batch-16 shape: ragged prefixes, active keys folded into
    # the last chunk, XCD-aligned mapping
    lens = [2176 - 37 * s for s in range(16)]
    bias = dict(prefix=_steps([0, 10, 2, 20], 512), active=_const(21.0))
    _check_biased(99, 16, 32, 32, 8, 128, "bf16", lens, [0, 32], BIDIR, bias, cap=2176)


@pytest.mark.parametrize("N", [4, 16, 64])
@pytest.mark.parametrize("mode", [BIDIR, CAUSAL])
def test_running_max_jumps_fork(N, mode):
    # N = 4: split plan; 16: row-tile form with key splits; 64: row-tile form,
    # one split, the two key halves merged in LDS
    priv = [(13 * s + 5) % 48 for s in range(N)]
    bias = dict(prefix=PREFIX_JUMPS, priv=_const(21.0), active=_const(22.0))
    _check_biased(100 + N, N, 24, 16, 2, 128, "bf16", [3282], [0, 9, 24], mode, bias, fork=True,
                  priv_len=priv, priv_cap=48)


@pytest.mark.parametrize("splits", [0, 1, 3])
def test_running_max_jumps_fp32(splits):
    bias = dict(prefix=_steps([0, 9, 1, 18], 64), active=_const(16.0))
    _check_biased(110 + splits, 1, 8, 4, 1, 64, "f32", [256], [0, 8], BIDIR, bias, n_splits=splits)


# ---- query heads per KV head that are not powers of two (12q/2kv, 28q/4kv
# and the like): the kernels split row indices by the group size through a
# multiply-high (tests/test_fastdiv.py checks its constants on the CPU)


@pytest.mark.parametrize("group", [3, 5, 6, 7, 12, 16])
@pytest.mark.parametrize("mode", [BIDIR, CAUSAL])
def test_odd_group_sizes(group, mode):
    _check(120 + group, 1, 20, 2 * group, 2, 128, "bf16", [777], [0, 7, 20], mode, cap=800)


@pytest.mark.parametrize("group", [3, 7])
def test_odd_group_sizes_two_column_tiles(group):
    # 300 rows x group 7 = 2100 rows per group: 128-row tiles, compact records
    _check(130 + group, 1, 300, 4 * group, 4, 64, "bf16", [500], [0, 100, 300], CAUSAL)


@pytest.mark.parametrize("group", [5, 6, 7])
@pytest.mark.parametrize("mode", [BIDIR, CAUSAL])
def test_odd_group_sizes_fork_row_tiles(group, mode):
    # 64 rollouts: half of a rollout's 24 x group rows (60 / 72 / 84) fills one
    # 96-row tile of the row-tile form, one key split
    priv = [(5 * s) % 40 for s in range(64)]
    _check(140 + group, 64, 24, 2 * group, 2, 128, "bf16", [1500], [0, 10, 24], mode, fork=True,
           priv_len=priv, priv_cap=40)


@pytest.mark.parametrize("N,group", [(16, 6), (16, 3), (4, 7)])
def test_odd_group_sizes_fork(N, group):
    # N = 16, group 6: row-tile form with key splits; group 3 and N = 4: split plan
    priv = [(7 * s + 3) % 48 for s in range(N)]
    _check(150 + N + group, N, 24, 2 * group, 2, 128, "bf16", [3282], [0, 24], CAUSAL, fork=True,
           priv_len=priv, priv_cap=48)


def test_odd_group_sizes_batch():
    # 12 sequences x 28q/4kv, ragged prefixes
    lens = [900 - 61 * s for s in range(12)]
    _check(160, 12, 16, 28, 4, 128, "bf16", lens, [0, 5, 16], BIDIR, cap=900)


@pytest.mark.parametrize("group", [3, 6])
def test_odd_group_sizes_fp32(group):
    _check(170 + group, 1, 8, group, 1, 64, "f32", [256], [0, 3, 8], CAUSAL)
