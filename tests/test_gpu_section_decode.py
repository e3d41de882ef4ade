"""A whole Section Diffusion decode on the GPU (Fast-dDrive method summary,
sec. 3.1 - 3.2) against the float64 schedule oracle on the same seeded
inputs: the tokens of every row (scaffold rows keep their template tokens),
sampled steps' attention outputs, and the cache the commits leave.  Block
visibility and section visibility (the blocks of a section attend to one
another and the section is committed whole), with and without the scaffold
rows inside the blocks."""

import numpy as np
import pytest

from oracle import section as OS
from tests import gpu_util as G
from block_causal_attention_gqa_amd import synth

pytestmark = pytest.mark.gpu

SEED = 4


@pytest.fixture(scope="module", autouse=True)
def _lib():
    G.require_lib()


def _layout(preset):
    """(blocks, blocks per section, editable mask, template tokens) the
    workload generator gives for the preset."""
    if preset.get("scaffold"):
        lay = synth.section_layout(preset["layout_seed"])
        blocks = [b for sec in lay for b in sec["blocks"]]
        editable = np.concatenate([sec["kinds"] for sec in lay])
        tmpl = synth.scaffold_tokens(preset["layout_seed"], len(editable), preset["vocab"])
        return blocks, [len(sec["blocks"]) for sec in lay], editable, np.where(editable == 0, tmpl, -1)
    n = sum(preset["blocks"])
    return list(preset["blocks"]), list(preset["sections"]), np.ones(n, np.uint8), np.full(n, -1)


@pytest.mark.parametrize("name,visibility,vocab", [
    ("section_scaffold", "section", None),     # full vocabulary
    ("section_scaffold", "block", 32768),
    ("section", "section", 32768),
    ("section", "block", None),                # the timed shapes, full vocabulary
])
def test_section_decode_matches_oracle(name, visibility, vocab):
    import torch
    from block_causal_attention_gqa_amd import decode
    print("section decode %s visibility=%s vocab=%s" % (name, visibility, vocab), flush=True)
    p = dict(synth.PRESETS[name])
    if vocab:
        p["vocab"] = vocab
    blocks, per_section, editable, template = _layout(p)
    if visibility == "section":
        first = np.concatenate([[0], np.cumsum(per_section)])
        units = [list(range(first[i], first[i + 1])) for i in range(len(per_section))]
    else:
        units = [[b] for b in range(len(blocks))]
    unit_rows = {b: sum(blocks[x] for x in u) for u in units for b in u}
    Hq, Hkv, D, steps = p["n_q_heads"], p["n_kv_heads"], p["head_dim"], p["steps"]
    frac = 0.2

    def inputs(b, st):
        (_, q), (_, k), (_, v) = synth.active_qkv(SEED, 1, unit_rows[b], Hq, Hkv, D, p["dtype"], b, st)
        lg = synth.logits(SEED, blocks[b], p["vocab"], p["sigma"], b, st)
        synth.plant_peaks(lg, SEED, frac, 12.0, b, st)
        return q, k, v, lg

    nb = len(blocks)
    widest = max(range(nb), key=lambda b: unit_rows[b])
    sample = {(0, 0), (widest, steps - 1), (nb // 2, 3), (nb - 1, steps - 1)}
    cap = p["prefix"] + sum(blocks)
    (_, _), (pk, pv) = synth.kv_cache(SEED, 1, Hkv, cap, D, [p["prefix"]], p["dtype"])
    want = OS.section_decode(pk[0], pv[0], p["prefix"], units, blocks, inputs, steps, p["threshold"], editable,
                             template, scale=D ** -0.5, keep=sample, attend_all=False)

    dec = decode.SectionDecode(p, seed=SEED, device=G.DEV, planted_frac=frac, visibility=visibility)
    seen = {}

    def after_attn(b, st, out):
        if (b, st) in sample:
            torch.cuda.synchronize()
            seen[(b, st)] = out.float().cpu().numpy()

    dec.after_attn = after_attn
    dec.run()
    torch.cuda.synchronize()
    assert dec.blocks == blocks
    assert np.array_equal(dec.tokens.cpu().numpy(), want["tokens"])
    assert not dec.masked.cpu().numpy().any() and not want["masked"].any()
    for key in sample:
        err = np.abs(seen[key] - want["attention"][key]).max()
        assert err <= 1e-2, "block %d step %d: attention max-abs %.3g" % (key[0], key[1], err)
    n = want["cache_k"].shape[1]
    assert n == cap
    assert np.array_equal(dec.cache.k[0].float().cpu().numpy(), want["cache_k"])
    assert np.array_equal(dec.cache.v[0].float().cpu().numpy(), want["cache_v"])
    assert dec.tokens_per_decode == int(editable.sum())
