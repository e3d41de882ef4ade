"""Captured HIP graphs of whole decodes against the float64 oracle and
against the eager calls.  The bench times the section decode as one captured
graph, so every launch's arguments (cache lengths, block offsets, workspace)
must be baked in correctly and nothing may depend on state that only the
eager run sets up.  Each replay follows eager work that scrambles the
outputs, the cache rows the decode commits and the workspaces, with
synchronisations in between; every replay's tokens, masks and committed cache
must equal the oracle's section decode on the same seeded inputs (the bench's
own workload among them, full vocabulary) and the eager run bit for bit."""

import numpy as np
import pytest
import torch

from oracle import attention as OA, section as OS, unmask as OU, verify as OV
from tests import gpu_util as G
from block_causal_attention_gqa_amd import decode, synth

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _lib():
    G.require_lib()


def _capture(fn, stream):
    with torch.cuda.stream(stream):
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn()
    torch.cuda.synchronize()
    return g


def oracle_section(p, seed, planted_frac=0.0):
    """The oracle's block-visibility section decode of one sequence on the
    inputs SectionDecode(p, seed, planted_frac=...) draws (attention outputs
    are not needed: the synthetic logits do not depend on them)."""
    blocks = list(p["blocks"])
    n = sum(blocks)
    Hq, Hkv, D = p["n_q_heads"], p["n_kv_heads"], p["head_dim"]

    def inputs(b, st):
        (_, q), (_, k), (_, v) = synth.active_qkv(seed, 1, blocks[b], Hq, Hkv, D, p["dtype"], b, st)
        lg = synth.logits(seed, blocks[b], p["vocab"], p["sigma"], b, st)
        if planted_frac:
            synth.plant_peaks(lg, seed, planted_frac, 12.0, b, st)
        return q, k, v, lg

    _, (pk, pv) = synth.kv_cache(seed, 1, Hkv, p["prefix"] + n, D, [p["prefix"]], p["dtype"])
    return OS.section_decode(pk[0], pv[0], p["prefix"], [[b] for b in range(len(blocks))], blocks, inputs,
                             p["steps"], p["threshold"], np.ones(n, np.uint8), np.full(n, -1, np.int32),
                             scale=D ** -0.5, attend_all=False)


def _check_oracle(dec, want, what):
    assert np.array_equal(dec.tokens.cpu().numpy(), want["tokens"]), "%s: tokens differ from the oracle" % what
    assert np.array_equal(dec.masked.cpu().numpy(), want["masked"]), "%s: masks differ from the oracle" % what
    assert np.array_equal(dec.cache.k[0].float().cpu().numpy(), want["cache_k"]), "%s: cache k" % what
    assert np.array_equal(dec.cache.v[0].float().cpu().numpy(), want["cache_v"]), "%s: cache v" % what


@pytest.mark.parametrize("seed,vocab,planted", [(5, 32768, 0.2), (0, None, 0.0)])
def test_section_decode_graph_replays_match_oracle_and_eager(seed, vocab, planted):
    # (0, full vocabulary, no planted rows) is the bench's own workload
    p = dict(synth.PRESETS["section"])
    if vocab:
        p["vocab"] = vocab
    print("graph: section decode, %d blocks, vocab %d, seed %d" % (len(p["blocks"]), p["vocab"], seed), flush=True)
    want_oracle = oracle_section(p, seed, planted)
    dec = decode.SectionDecode(p, seed=seed, device=G.DEV, planted_frac=planted)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        dec.run()
    torch.cuda.synchronize()
    want = [t.clone() for t in (dec.tokens, dec.masked, dec.cache.k, dec.cache.v)]
    assert not want[1].any()
    _check_oracle(dec, want_oracle, "eager decode")
    g = _capture(dec.run, stream)
    len0 = int(dec.len0[0])
    gen = torch.Generator(device=G.DEV).manual_seed(0)
    for i in range(REPLAYS):
        # eager work between replays: scramble what the decode writes
        dec.tokens.fill_(-7)
        dec.masked.fill_(1)
        for c in (dec.cache.k, dec.cache.v):
            c[:, :, len0:] = torch.randn(c[:, :, len0:].shape, generator=gen, device=G.DEV).to(c.dtype)
        dec.ws_attn.fill_(0xAB)
        dec.ws_unmask.fill_(0xCD)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        _check_oracle(dec, want_oracle, "replay %d" % i)
        got = (dec.tokens, dec.masked, dec.cache.k, dec.cache.v)
        for name, a, b in zip(("tokens", "masked", "cache k", "cache v"), got, want):
            assert torch.equal(a, b), "replay %d: %s differs from the eager decode" % (i, name)


def oracle_fork_round(fv, seed, block):
    """The oracle's fork round on ForkVerify's inputs: the verify pass's
    attention, the draft tokens and masks, the accept lengths and bonuses."""
    h = fv.host_inputs(seed=seed, block=block)
    N, R = fv.N, fv.R
    q, k, v = h["qkv"][1]
    attn = OA.attention_step(q, h["pk"], h["pv"], [fv.prefix], k, v, [0, R], OA.MASK_CAUSAL, scale=fv.scale,
                             priv_k=h["vk"], priv_v=h["vv"], priv_len=fv.priv_len)
    masked0 = (1 - h["fixed"]).reshape(-1).astype(np.uint8)
    m, t, _, _ = OU.unmask_select(h["draft_logits"], fv.blk_rows, [OU.MODE_SEMI] * N, [1] * N, np.float32(0.0),
                                  masked0, h["tokens0"])
    if fv.temperature is None:
        acc, bon = OV.spec_verify(h["verify_logits"], t.reshape(N, R), h["fixed"], np.zeros(N, np.int32))
    else:
        acc, bon = OV.spec_verify_sampled(h["verify_logits"], h["noise"], 1.0 / fv.temperature, t.reshape(N, R),
                                          h["fixed"], np.zeros(N, np.int32))
    return attn, t, m, acc, bon


@pytest.mark.parametrize("temperature", [None, 0.7])
def test_fork_round_graph_replays_match_oracle_and_eager(temperature):
    N = 16
    print("graph: fork round N=%d temperature=%s" % (N, temperature), flush=True)
    fv = decode.ForkVerify(N, seed=6, device=G.DEV, block=0, temperature=temperature,
                           preset=dict(synth.PRESETS["fork"], vocab=20000))
    w_attn, w_tok, w_masked, w_acc, w_bon = oracle_fork_round(fv, 6, 0)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        fv.run()
    torch.cuda.synchronize()
    want = [t.clone() for t in (fv.out, fv.tokens, fv.masked, fv.accept_len, fv.bonus)]
    g = _capture(fv.run, stream)
    for i in range(REPLAYS):
        fv.out.fill_(3.0)
        fv.tokens.fill_(-9)
        fv.masked.fill_(0)
        fv.accept_len.fill_(-1)
        fv.bonus.fill_(-1)
        fv.ws_attn.fill_(0x7F)
        fv.ws_verify.fill_(0x11)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        got = (fv.out, fv.tokens, fv.masked, fv.accept_len, fv.bonus)
        for name, a, b in zip(("attention out", "tokens", "masked", "accept_len", "bonus"), got, want):
            assert torch.equal(a, b), "replay %d: %s differs from the eager round" % (i, name)
        err = np.abs(fv.out.float().cpu().numpy() - w_attn).max()
        assert err <= 1e-2, "replay %d: verify-pass attention max-abs %.3g against the oracle" % (i, err)
        assert np.array_equal(fv.tokens.cpu().numpy(), w_tok) and np.array_equal(fv.masked.cpu().numpy(), w_masked)
        assert np.array_equal(fv.accept_len.cpu().numpy(), w_acc) and np.array_equal(fv.bonus.cpu().numpy(), w_bon)
    assert np.all(fv.accept_len.cpu().numpy() >= 0)
