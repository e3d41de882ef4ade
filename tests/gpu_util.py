"""Helpers for the GPU parity tests: move seeded synthetic inputs to the
device, run the library through the binding, and read results back."""

import numpy as np
import torch

from block_causal_attention_gqa_amd import binding as B
from block_causal_attention_gqa_amd import synth

DEV = "cuda:0"


def require_lib():
    B.lib()
    assert torch.cuda.is_available(), "the GPU tests need a GPU"


def attn_case(seed, S, R, Hq, Hkv, D, dtype, prefix_len, blk_off, mode, cap=None,
              fork=False, priv_len=None, priv_cap=None, n_splits=0, scale=None, key_bias=None):
    """Run bc_attn_step on seeded inputs; return (gpu_out f64, host inputs).

    key_bias: optional dict of functions ("prefix", "priv", "active") from
    key positions (an int array) to score offsets; see biased_keys."""
    cap = cap or max(max(prefix_len), 1)
    Sp = 1 if fork else S
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    (pk_t, pv_t), (pk, pv) = synth.kv_cache(seed, Sp, Hkv, cap, D, prefix_len, dtype)
    (q_t, q), (k_t, k), (v_t, v) = synth.active_qkv(seed, S, R, Hq, Hkv, D, dtype, 0)
    vk_t = vv_t = vk = vv = None
    if fork:
        priv_cap = priv_cap or max(max(priv_len), 1)
        (vk_t, vv_t), (vk, vv) = synth.kv_cache(seed, S, Hkv, priv_cap, D, priv_len, dtype,
                                                purpose=("priv_k", "priv_v"))
    if key_bias is not None:
        u = synth.normal(seed, "score_dir", (D,)).astype(np.float64)
        u /= np.linalg.norm(u)
        q_t, q = synth.to_dtype((q + u / scale).astype(np.float32), dtype)
        f = key_bias.get("prefix")
        if f is not None:
            pk_t, pk = biased_keys(pk, [int(n) for n in prefix_len], f, u, dtype)
        f = key_bias.get("active")
        if f is not None:
            k_t, k = biased_keys(k, [R] * S, f, u, dtype)
        f = key_bias.get("priv")
        if fork and f is not None:
            vk_t, vk = biased_keys(vk, [int(n) for n in priv_len], f, u, dtype)
    prefix = B.KVCache(pk_t.to(DEV), pv_t.to(DEV))
    priv = B.KVCache(vk_t.to(DEV), vv_t.to(DEV)) if fork else None
    tdt = synth.torch_dtype(dtype)
    out = torch.empty((S, R, Hq, D), dtype=tdt, device=DEV)
    nb = B.bc_attn_workspace_bytes(prefix, priv, (S, R, Hq, D), blk_off, n_splits)
    assert nb > 0
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    B.bc_attn_step(prefix, prefix_len, priv, priv_len, q_t.to(DEV), k_t.to(DEV), v_t.to(DEV),
                   blk_off, mode, scale, out, ws, n_prefix_splits=n_splits)
    torch.cuda.synchronize()
    host = dict(q=q, pk=pk, pv=pv, k=k, v=v, vk=vk, vv=vv, scale=scale)
    return out.float().cpu().numpy().astype(np.float64), host


def biased_keys(k, lengths, fn, u, dtype):
    """Keys [S][Hkv][n][D] with b(j) u added to key j < lengths[s] of every
    sequence and head (u a unit vector, b = fn(j)), rounded to dtype.  With
    every query shifted by u / scale, the scaled score of key j rises by about
    b(j), so chosen positions can raise a row's running maximum by a chosen
    amount.  Returns (torch CPU tensor, float32 array of the rounded values)."""
    x = k.astype(np.float64).copy()
    for s, n in enumerate(lengths):
        if n > 0:
            b = np.asarray(fn(np.arange(n)), np.float64)
            x[s, :, :n, :] += b[None, :, None] * u[None, None, :]
    return synth.to_dtype(x.astype(np.float32), dtype)


def to_dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)
