"""The WAM-Diff2-shaped large-block decode on the GPU (WAM-Diff2 article
sec. 2.1: the block size B is the dial between AR and diffusion decoding, and
B = 1 is standard AR decoding; sec. 3: accuracy saturates at 8-16 denoise
steps), against the float64 section-decode oracle on the same seeded inputs:
32 query / 8 KV heads, head_dim 128, bf16, a 2048-token prefix, 256 output
tokens.

* block size 32 with 16 steps per block at batch 1 and at batch 16 with
  independent seeded prefixes: every sequence's tokens and committed cache bit
  for bit, sampled steps' attention within 1e-2;
* the block-size sweep B = 1, 4, 8, 16, 32 (256 / B blocks, min(16, B)
  steps) at batch 1, the same checks;
* B = 1 is causal decoding: the decode with bidirectional blocks and the
  decode with causal blocks produce the same attention outputs, tokens and
  cache bit for bit, and every step's output matches the cache-free causal
  attention over the whole sequence (prefix and the 256 decoded positions)."""

import numpy as np
import pytest

from oracle import attention as OA, section as OS
from tests import gpu_util as G
from block_causal_attention_gqa_amd import synth

pytestmark = pytest.mark.gpu

SEED = 21


@pytest.fixture(scope="module", autouse=True)
def _lib():
    G.require_lib()


def _inputs(p, seed, S, planted_frac):
    """Every (block, step)'s host inputs of all S sequences, as SectionDecode
    draws them: (q, k, v) float32 and the logits [S * rows][V]."""
    Hq, Hkv, D = p["n_q_heads"], p["n_kv_heads"], p["head_dim"]
    out = {}
    for b, bs in enumerate(p["blocks"]):
        for st in range(p["steps"]):
            (_, q), (_, k), (_, v) = synth.active_qkv(seed, S, bs, Hq, Hkv, D, p["dtype"], b, st)
            lg = synth.logits(seed, S * bs, p["vocab"], p["sigma"], b, st)
            if planted_frac:
                synth.plant_peaks(lg, seed, planted_frac, 12.0, b, st)
            out[(b, st)] = (q, k, v, lg)
    return out


def _oracle_seq(p, seed, S, s, inputs, keep):
    """The oracle's block-visibility decode of sequence s of the batch."""
    blocks = list(p["blocks"])
    n = sum(blocks)
    Hkv, D = p["n_kv_heads"], p["head_dim"]
    _, (pk, pv) = synth.kv_cache(seed, S, Hkv, p["prefix"] + n, D, [p["prefix"]] * S, p["dtype"])

    def inp(b, st):
        q, k, v, lg = inputs[(b, st)]
        bs = blocks[b]
        return q[s:s + 1], k[s:s + 1], v[s:s + 1], lg[s * bs:(s + 1) * bs]

    return OS.section_decode(pk[s], pv[s], p["prefix"], [[b] for b in range(len(blocks))], blocks, inp,
                             p["steps"], p["threshold"], np.ones(n, np.uint8), np.full(n, -1, np.int32),
                             scale=D ** -0.5, keep=keep, attend_all=False)


def _run_and_check(p, S, planted_frac=0.2):
    import torch
    from block_causal_attention_gqa_amd import decode
    blocks, steps = list(p["blocks"]), p["steps"]
    nb = len(blocks)
    keep = {(0, 0), (nb // 2, steps // 2), (nb - 1, steps - 1)}
    dec = decode.SectionDecode(p, seed=SEED, n_seq=S, device=G.DEV, planted_frac=planted_frac)
    seen = {}

    def after_attn(b, st, out):
        if (b, st) in keep:
            torch.cuda.synchronize()
            seen[(b, st)] = out.float().cpu().numpy()

    dec.after_attn = after_attn
    dec.run()
    torch.cuda.synchronize()
    inputs = _inputs(p, SEED, S, planted_frac)
    tokens = dec.tokens.cpu().numpy()
    kc = dec.cache.k.float().cpu().numpy()
    vc = dec.cache.v.float().cpu().numpy()
    row0 = np.concatenate([[0], np.cumsum(blocks)])
    for s in range(S):
        want = _oracle_seq(p, SEED, S, s, inputs, keep)
        # the device rows are laid out [block][sequence][row]
        got = np.concatenate([tokens[S * row0[b] + s * bs: S * row0[b] + (s + 1) * bs] for b, bs in enumerate(blocks)])
        assert np.array_equal(got, want["tokens"]), "sequence %d: tokens" % s
        assert np.array_equal(kc[s], want["cache_k"]) and np.array_equal(vc[s], want["cache_v"]), \
            "sequence %d: cache" % s
        for key in keep:
            err = np.abs(seen[key][s] - want["attention"][key][0]).max()
            assert err <= 1e-2, "sequence %d block %d step %d: attention max-abs %.3g" % (s, key[0], key[1], err)
    assert not dec.masked.cpu().numpy().any()
    return dec


@pytest.mark.parametrize("S", [1, 16])
def test_large_block_batch_matches_oracle(S):
    print("large-block decode B=32 batch %d" % S, flush=True)
    _run_and_check(synth.large_block_preset(32, n_seq=S, vocab=2048), S)


@pytest.mark.parametrize("B", synth.LARGE_BLOCK_SIZES)
def test_block_size_sweep_matches_oracle(B):
    print("large-block decode sweep B=%d" % B, flush=True)
    dec = _run_and_check(synth.large_block_preset(B, vocab=4096), 1)
    assert dec.denoise_steps == (256 // B) * min(16, B)


def test_block_size_one_is_causal_decoding():
    import torch
    from block_causal_attention_gqa_amd import binding as B, decode
    print("large-block decode B=1: bidirectional vs causal blocks vs full causal recompute", flush=True)
    p = synth.large_block_preset(1, vocab=1024)
    runs = {}
    for mask in (B.BC_MASK_BLOCK_BIDIR, B.BC_MASK_BLOCK_CAUSAL):
        dec = decode.SectionDecode(p, seed=SEED, device=G.DEV, planted_frac=0.2, mask=mask)
        outs = []

        def after_attn(b, st, out):
            outs.append(out.clone())

        dec.after_attn = after_attn
        dec.run()
        torch.cuda.synchronize()
        runs[mask] = (torch.stack(outs).cpu(), dec.tokens.cpu(), dec.cache.k.cpu(), dec.cache.v.cpu())
    a, c = runs[B.BC_MASK_BLOCK_BIDIR], runs[B.BC_MASK_BLOCK_CAUSAL]
    for name, x, y in zip(("attention", "tokens", "cache k", "cache v"), a, c):
        assert torch.equal(x, y), "B = 1: %s differs between bidirectional and causal blocks" % name

    # every step against the cache-free causal attention over the whole
    # sequence: position 2048 + i holds the query and the K/V of block i
    Hq, Hkv, D, L0 = p["n_q_heads"], p["n_kv_heads"], p["head_dim"], p["prefix"]
    n = len(p["blocks"])
    _, (pk, pv) = synth.kv_cache(SEED, 1, Hkv, L0 + n, D, [L0], p["dtype"])
    q = np.zeros((L0 + n, Hq, D), np.float32)
    k = np.concatenate([pk[0, :, :L0].transpose(1, 0, 2), np.zeros((n, Hkv, D), np.float32)])
    v = np.concatenate([pv[0, :, :L0].transpose(1, 0, 2), np.zeros((n, Hkv, D), np.float32)])
    for i in range(n):
        (_, qi), (_, ki), (_, vi) = synth.active_qkv(SEED, 1, 1, Hq, Hkv, D, p["dtype"], i, 0)
        q[L0 + i], k[L0 + i], v[L0 + i] = qi[0, 0], ki[0, :, 0], vi[0, :, 0]
    full = OA.full_sequence_attention(q, k, v, np.arange(L0 + n), OA.MASK_CAUSAL, scale=D ** -0.5)
    got = a[0].float().numpy().reshape(n, Hq, D)
    err = np.abs(got - full[L0:]).max()
    assert err <= 1e-2, "B = 1 decode vs full causal recompute: max-abs %.3g" % err


def test_bench_configuration_sampled_sequences_match_oracle():
    """The large-block decode as the bench times it: batch 16, B = 32,
    vocabulary 151936, 4 distinct logits and Q/K/V sets cycled over the
    steps, seed 0.  Two of the 16 sequences (the first and the twelfth; the
    oracle's float64 decode of a sequence at this vocabulary takes several
    seconds) are decoded by the oracle on the same pool entries: tokens and
    committed cache bit for bit, and the attention of the step the bench
    times alone (the middle block's first step) within 1e-2."""
    import torch
    from block_causal_attention_gqa_amd import decode
    print("large-block decode B=32 batch 16 vocab 151936 (bench configuration)", flush=True)
    S, seed, pool = 16, 0, 4
    p = synth.large_block_preset(32, n_seq=S)
    blocks, steps, V = list(p["blocks"]), p["steps"], p["vocab"]
    Hq, Hkv, D = p["n_q_heads"], p["n_kv_heads"], p["head_dim"]
    dec = decode.SectionDecode(p, seed=seed, n_seq=S, device=G.DEV, logits_pool=pool, qkv_pool=pool)
    keep = {(len(blocks) // 2, 0)}
    seen = {}

    def after_attn(b, st, out):
        if (b, st) in keep:
            torch.cuda.synchronize()
            seen[(b, st)] = out.float().cpu().numpy()

    dec.after_attn = after_attn
    dec.run()
    torch.cuda.synchronize()
    tokens = dec.tokens.cpu().numpy()
    kc = dec.cache.k.float().cpu().numpy()
    vc = dec.cache.v.float().cpu().numpy()
    assert not dec.masked.cpu().numpy().any()
    # the pools as the decoder draws them (the same seeded generators)
    lg_pool = [synth.logits(seed, S * 32, V, p["sigma"], 1000 + i) for i in range(pool)]
    qkv_pool = [synth.active_qkv(seed, S, 32, Hq, Hkv, D, p["dtype"], 2000 + 32, i) for i in range(pool)]
    _, (pk, pv) = synth.kv_cache(seed, S, Hkv, p["prefix"] + sum(blocks), D, [p["prefix"]] * S, p["dtype"])
    row0 = np.concatenate([[0], np.cumsum(blocks)])
    for s in (0, 11):
        def inp(b, st):
            i = (b * steps + st) % pool
            (_, q), (_, k), (_, v) = qkv_pool[i]
            return q[s:s + 1], k[s:s + 1], v[s:s + 1], lg_pool[i][s * 32:(s + 1) * 32]

        n = sum(blocks)
        want = OS.section_decode(pk[s], pv[s], p["prefix"], [[b] for b in range(len(blocks))], blocks, inp, steps,
                                 p["threshold"], np.ones(n, np.uint8), np.full(n, -1, np.int32), scale=D ** -0.5,
                                 keep=keep, attend_all=False)
        got = np.concatenate([tokens[S * row0[b] + s * bs: S * row0[b] + (s + 1) * bs] for b, bs in enumerate(blocks)])
        assert np.array_equal(got, want["tokens"]), "sequence %d: tokens" % s
        assert np.array_equal(kc[s], want["cache_k"]) and np.array_equal(vc[s], want["cache_v"]), "sequence %d: cache" % s
        for key in keep:
            err = np.abs(seen[key][s] - want["attention"][key][0]).max()
            assert err <= 1e-2, "sequence %d: attention max-abs %.3g" % (s, err)
