"""Seeded synthetic inputs shaped like the pages' workloads.

This module is shared by the tests, ``bench.py`` and the smoke check, and feeds
both the HIP library and the CPU oracle with the same arrays.  It only draws
random numbers and lays out shapes; it computes nothing the decoding step
computes (no softmax, no argmax, no masks).

Every draw comes from its own NumPy PCG64 stream keyed by
(seed, purpose, *indices) through ``numpy.random.SeedSequence``, so any one
tensor can be regenerated independently of the others.

bf16 values are produced by rounding float32 draws to nearest-even once on the
host (through torch's dtype conversion); the float32 upcast of the rounded
values is exact and is what the oracle reads.
"""

import numpy as np
import torch

# purpose tags for SeedSequence keys
_TAGS = {
    "prefix_k": 1, "prefix_v": 2, "q": 3, "k": 4, "v": 5, "logits": 6,
    "priv_k": 7, "priv_v": 8, "draft": 9, "peak": 10, "ratio": 11,
    "subset": 12, "commit_k": 13, "commit_v": 14, "misc": 15, "gumbel": 16,
    "layout": 17, "scaffold": 18, "score_dir": 19,
}


def rng(seed, purpose, *idx):
    """Independent generator for one tensor."""
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([int(seed), _TAGS[purpose]] + [int(i) for i in idx])))


def normal(seed, purpose, shape, *idx, sigma=1.0):
    return (rng(seed, purpose, *idx).standard_normal(shape) * sigma).astype(np.float32)


def to_dtype(x_f32, dtype):
    """Round a float32 array to ``dtype`` ("f32" or "bf16").

    Returns (torch CPU tensor of that dtype, float32 NumPy array holding the
    exactly-representable rounded values)."""
    t = torch.from_numpy(np.ascontiguousarray(x_f32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
        return t, t.to(torch.float32).numpy()
    if dtype == "f32":
        return t.clone(), x_f32.copy()
    raise ValueError(dtype)


def torch_dtype(dtype):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


# ---------------------------------------------------------------------------
# Workload presets.  Sizes follow the configurations the pages' systems run:
#   tiny       : 1 seq, 4q/1kv heads, D 64, fp32, prefix 256, one block of 8,
#                logits [8 x 1024] ~ N(0, 3^2), threshold 0.9, >= 1 commit/step
#   section    : Fast-dDrive section decode, bs1, 16q/2kv, D 128, bf16,
#                prefix 3072, editable sections 12/192/6/70 in blocks of 32,
#                8 denoise steps per block, logits [b x 151936] ~ N(0, 4^2)
#   large_block: WAM-Diff2 large-block decode, 32q/8kv, D 128, bf16,
#                prefix 2048, 8 blocks of 32, 16 steps per block, batch 1/16
#   pipelined  : Fast-dVLA, 16q/2kv, D 128, bf16, prefix 512, 3 active blocks
#                of 7, logits [21 x 2048]; variant 625 tokens in blocks of 32
#   section_scaffold: the section decode with the sections' scaffold tokens
#                inside the blocks (404 rows, blocks of <= 32 editable rows)
#   fork       : shared prefix 3072 + 210, 16q/2kv, D 128, bf16, N rollouts,
#                trajectory blocks 24/23/23, logits [24 x 151936]; a planted
#                argmax 1.0 above the 7 sigma clip in the trajectory rounds
# ---------------------------------------------------------------------------

SECTION_EDITABLE = {"critical_objects": 12, "explanation": 192,
                    "future_meta_behavior": 6, "trajectory": 70}
SECTION_ORDER = ["critical_objects", "explanation", "future_meta_behavior", "trajectory"]
# scaffold (template) tokens of each section, from the same table
SECTION_SCAFFOLD = {"critical_objects": 80, "explanation": 6,
                    "future_meta_behavior": 18, "trajectory": 20}


def split_sizes(n, d):
    """Cut n editable tokens into consecutive blocks of d with a final
    partial block (the n // d full blocks first)."""
    sizes = [d] * (n // d)
    if n % d:
        sizes.append(n % d)
    return sizes


def section_layout(seed, d=32):
    """Output rows of the four sections with their scaffold tokens inside
    the blocks.  Each section's rows are a seeded interleaving of its
    editable and scaffold counts (the pages give the counts, not the
    order); a block ends right after every d-th editable row while editable
    rows remain, so the last block of a section also takes its trailing
    scaffold.  Returns one dict per section, in decoding order:
    ``kinds`` (uint8 [rows], 1 = editable, 0 = scaffold) and ``blocks``
    (rows per block)."""
    out = []
    for i, name in enumerate(SECTION_ORDER):
        ne, ns = SECTION_EDITABLE[name], SECTION_SCAFFOLD[name]
        kinds = np.zeros(ne + ns, np.uint8)
        kinds[rng(seed, "layout", i).permutation(ne + ns)[:ne]] = 1
        blocks, start, seen = [], 0, 0
        for r in range(ne + ns):
            seen += int(kinds[r])
            if kinds[r] and seen % d == 0 and seen < ne:
                blocks.append(r + 1 - start)
                start = r + 1
        blocks.append(ne + ns - start)
        out.append(dict(name=name, kinds=kinds, blocks=blocks))
    return out


def scaffold_tokens(seed, n, vocab, *idx):
    """Token ids of prefilled scaffold rows (uniform over the vocabulary)."""
    return rng(seed, "scaffold", *idx).integers(0, vocab, size=n).astype(np.int32)


PRESETS = {
    "tiny": dict(n_seq=1, n_q_heads=4, n_kv_heads=1, head_dim=64, dtype="f32",
                 prefix=256, blocks=[8], steps=1, vocab=1024, sigma=3.0,
                 threshold=0.9),
    "section": dict(n_seq=1, n_q_heads=16, n_kv_heads=2, head_dim=128, dtype="bf16",
                    prefix=3072,
                    blocks=sum((split_sizes(SECTION_EDITABLE[s], 32) for s in SECTION_ORDER), []),
                    sections=[len(split_sizes(SECTION_EDITABLE[s], 32)) for s in SECTION_ORDER],
                    steps=8, vocab=151936, sigma=4.0, threshold=0.9),
    # the same decode with the scaffold rows inside the blocks (404 rows:
    # 280 editable, 124 scaffold), the layout drawn once from layout_seed
    "section_scaffold": dict(n_seq=1, n_q_heads=16, n_kv_heads=2, head_dim=128, dtype="bf16",
                             prefix=3072, scaffold=True, layout_seed=0, steps=8, vocab=151936,
                             sigma=4.0, threshold=0.9),
    "large_block": dict(n_seq=1, n_q_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16",
                        prefix=2048, blocks=[32] * 8, steps=16, vocab=151936, sigma=4.0,
                        threshold=0.9),
    "pipelined": dict(n_seq=1, n_q_heads=16, n_kv_heads=2, head_dim=128, dtype="bf16",
                      prefix=512, blocks=[7, 7, 7], steps=None, vocab=2048, sigma=4.0,
                      threshold=0.9),
    "pipelined_625": dict(n_seq=1, n_q_heads=16, n_kv_heads=2, head_dim=128, dtype="bf16",
                          prefix=512, blocks=split_sizes(625, 32), window=3, vocab=2048,
                          sigma=4.0, threshold=0.9),
    "fork": dict(n_q_heads=16, n_kv_heads=2, head_dim=128, dtype="bf16",
                 prefix=3072 + 210, blocks=[24, 23, 23], vocab=151936, sigma=4.0, margin=1.0),
}


def large_block_preset(block_size, n_seq=1, vocab=None):
    """The WAM-Diff2-shaped large-block decode at block size B: 256 output
    tokens in 256 / B blocks of B, min(16, B) denoise steps per block."""
    p = dict(PRESETS["large_block"], n_seq=n_seq)
    p["blocks"] = [block_size] * (256 // block_size)
    p["steps"] = min(16, block_size)
    if vocab:
        p["vocab"] = vocab
    return p


LARGE_BLOCK_SIZES = (1, 4, 8, 16, 32)


def kv_cache(seed, n_seq, n_kv_heads, capacity, head_dim, lengths, dtype, purpose=("prefix_k", "prefix_v")):
    """A KV cache [S][Hkv][capacity][D] whose first lengths[s] rows hold
    N(0,1) draws and whose remaining rows are zero.  Returns
    ((k_t, v_t) torch CPU tensors, (k32, v32) float32 arrays)."""
    k = np.zeros((n_seq, n_kv_heads, capacity, head_dim), np.float32)
    v = np.zeros_like(k)
    for s in range(n_seq):
        n = int(lengths[s])
        k[s, :, :n] = normal(seed, purpose[0], (n_kv_heads, n, head_dim), s)
        v[s, :, :n] = normal(seed, purpose[1], (n_kv_heads, n, head_dim), s)
    kt, k32 = to_dtype(k, dtype)
    vt, v32 = to_dtype(v, dtype)
    return (kt, vt), (k32, v32)


def active_qkv(seed, n_seq, n_rows, n_q_heads, n_kv_heads, head_dim, dtype, *idx):
    """Active-row Q [S][R][Hq][D] and K/V [S][Hkv][R][D], N(0,1), redrawn per
    (idx...) because the model recomputes them every denoise step."""
    q = normal(seed, "q", (n_seq, n_rows, n_q_heads, head_dim), *idx)
    k = normal(seed, "k", (n_seq, n_kv_heads, n_rows, head_dim), *idx)
    v = normal(seed, "v", (n_seq, n_kv_heads, n_rows, head_dim), *idx)
    return to_dtype(q, dtype), to_dtype(k, dtype), to_dtype(v, dtype)


def logits(seed, n_rows, vocab, sigma, *idx):
    """float32 logits [R][V] ~ N(0, sigma^2)."""
    return normal(seed, "logits", (n_rows, vocab), *idx, sigma=sigma)


def plant_peaks(x, seed, frac, delta, *idx):
    """Raise one seeded token of a seeded fraction of rows by ``delta`` so that
    those rows carry a confident prediction (exercises the threshold branch).
    Modifies x in place and returns the list of (row, token) planted."""
    g = rng(seed, "peak", *idx)
    planted = []
    for r in range(x.shape[0]):
        if g.random() < frac:
            t = int(g.integers(x.shape[1]))
            x[r, t] += np.float32(delta)
            planted.append((r, t))
    return planted


def argmax_planted_logits(seed, n_rows, vocab, sigma, margin, *idx):
    """Logits whose row-wise argmax is known by construction: the draws are
    clipped to [-7 sigma, 7 sigma] and token t_r is set to 7 sigma + margin.
    Returns (logits, t)."""
    x = np.clip(logits(seed, n_rows, vocab, sigma, *idx), -7.0 * sigma, 7.0 * sigma)
    x = x.astype(np.float32)
    g = rng(seed, "peak", *idx)
    t = g.integers(0, vocab, size=n_rows).astype(np.int32)
    x[np.arange(n_rows), t] = np.float32(7.0 * sigma + margin)
    return x, t


def clipped_logits(seed, n, sigma, *idx):
    """float32 N(0, sigma^2) draws clipped to [-7 sigma, 7 sigma], flat [n]:
    the base of logits whose row argmax is then planted above 7 sigma."""
    x = rng(seed, "logits", *idx).standard_normal(n, dtype=np.float32)
    x *= np.float32(sigma)
    np.clip(x, np.float32(-7.0 * sigma), np.float32(7.0 * sigma), out=x)
    return x


def round_targets(seed, vocab, n_rows, *idx):
    """Seeded token ids [n_rows] planted as the row argmaxes of one round."""
    return rng(seed, "peak", *idx).integers(0, vocab, size=n_rows).astype(np.int32)


def drafts_with_agreement(seed, target, p_agree, vocab, *idx):
    """Draft tokens equal to ``target`` with probability p_agree per row, else
    a seeded different token."""
    g = rng(seed, "draft", *idx)
    d = np.array(target, dtype=np.int32).copy()
    for i in range(len(d)):
        if g.random() >= p_agree:
            alt = int(g.integers(vocab - 1))
            d[i] = alt if alt < target[i] else alt + 1
    return d


def gumbel(seed, shape, *idx):
    """float32 Gumbel(0, 1) noise, -log(-log U) with U uniform in (0, 1),
    for the sampled verify (the random numbers the method draws are inputs)."""
    u = rng(seed, "gumbel", *idx).random(shape)
    u = np.clip(u, np.finfo(np.float64).tiny, 1.0 - 2.0 ** -53)
    return (-np.log(-np.log(u))).astype(np.float32)
