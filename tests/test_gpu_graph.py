"""Captured HIP graphs of whole decodes replay exactly what the eager calls
compute.  The bench times the section decode as one captured graph, so every
launch's arguments (cache lengths, block offsets, workspace) must be baked in
correctly and nothing may depend on state that only the eager run sets up.
Each replay follows eager work that scrambles the outputs, the cache rows the
decode commits and the workspaces, with synchronisations in between, and must
match the eager result bit for bit."""

import numpy as np
import pytest
import torch

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


def test_section_decode_graph_replays_match_eager():
    p = dict(synth.PRESETS["section"], vocab=32768)
    print("graph: section decode, %d blocks, vocab %d" % (len(p["blocks"]), p["vocab"]), flush=True)
    dec = decode.SectionDecode(p, seed=5, device=G.DEV)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        dec.run()
    torch.cuda.synchronize()
    want = [t.clone() for t in (dec.tokens, dec.masked, dec.cache.k, dec.cache.v)]
    assert not want[1].any()
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
        got = (dec.tokens, dec.masked, dec.cache.k, dec.cache.v)
        for name, a, b in zip(("tokens", "masked", "cache k", "cache v"), got, want):
            assert torch.equal(a, b), "replay %d: %s differs from the eager decode" % (i, name)


@pytest.mark.parametrize("temperature", [None, 0.7])
def test_fork_round_graph_replays_match_eager(temperature):
    N = 16
    print("graph: fork round N=%d temperature=%s" % (N, temperature), flush=True)
    fv = decode.ForkVerify(N, seed=6, device=G.DEV, block=0, temperature=temperature,
                           preset=dict(synth.PRESETS["fork"], vocab=20000))
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
    assert np.all(fv.accept_len.cpu().numpy() >= 0)
