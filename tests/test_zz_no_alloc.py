"""The allocation-free attention entry point, bc_attn_step_static, against
bc_attn_step with a caller workspace, through the C ABI: two calls in a row
on the same device scratch (the second smaller than the first) must give the
same outputs bit for bit (the same kernels and the same split plan), and
within 1e-2 of the float64 oracle; a call whose split partials cannot fit in
the scratch is refused on the host with BC_ERR_SCRATCH, nothing launched."""

import numpy as np
import pytest
import torch

from oracle import attention as OA
from tests import gpu_util as G
from block_causal_attention_gqa_amd import binding as B, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    G.require_lib()


def _case(seed, S, R, Hq, Hkv, D, lens, blk_off, fork=False, priv_len=None):
    Sp = 1 if fork else S
    cap = max(lens)
    (pk_t, pv_t), (pk, pv) = synth.kv_cache(seed, Sp, Hkv, cap, D, lens, "bf16")
    (q_t, q), (k_t, k), (v_t, v) = synth.active_qkv(seed, S, R, Hq, Hkv, D, "bf16", 0)
    prefix = B.KVCache(pk_t.to(G.DEV), pv_t.to(G.DEV))
    priv = vk = vv = None
    if fork:
        (vk_t, vv_t), (vk, vv) = synth.kv_cache(seed, S, Hkv, max(max(priv_len), 1), D, priv_len, "bf16",
                                                purpose=("priv_k", "priv_v"))
        priv = B.KVCache(vk_t.to(G.DEV), vv_t.to(G.DEV))
    dev = dict(prefix=prefix, priv=priv, q=q_t.to(G.DEV), k=k_t.to(G.DEV), v=v_t.to(G.DEV))
    host = dict(q=q, pk=pk, pv=pv, k=k, v=v, vk=vk, vv=vv)
    return dev, host


CASES = [
    # (seed, S, R, Hq, Hkv, D, prefix lengths, blk_off, fork, priv_len, mask)
    (4, 64, 24, 16, 2, 128, [3282], [0, 9, 24], True, [(11 * s) % 48 for s in range(64)],
     B.BC_MASK_BLOCK_BIDIR),                                                          # fork, output written directly
    (5, 16, 32, 32, 8, 128, [2176 - 37 * s for s in range(16)], [0, 32], False, None,
     B.BC_MASK_BLOCK_BIDIR),                                                          # batch 16, folded, compact
    (1, 16, 24, 16, 2, 128, [3282], [0, 24], True, [24] * 16, B.BC_MASK_BLOCK_CAUSAL),  # fork, compact partials
    (2, 1, 32, 16, 2, 128, [3084], [0, 32], False, None, B.BC_MASK_BLOCK_BIDIR),         # bs1 section step
    (3, 1, 7, 16, 2, 64, [300], [0, 3, 7], False, None, B.BC_MASK_BLOCK_BIDIR),          # smaller, two blocks
]


def test_static_entry_matches_workspace_entry_on_consecutive_calls():
    for seed, S, R, Hq, Hkv, D, lens, off, fork, priv_len, mask in CASES:
        print("static attention: S=%d R=%d Hq=%d Hkv=%d D=%d prefix=%s fork=%s" % (S, R, Hq, Hkv, D, lens, fork),
              flush=True)
        dev, host = _case(seed, S, R, Hq, Hkv, D, lens, off, fork, priv_len)
        scale = D ** -0.5
        ws = torch.zeros(B.bc_attn_workspace_bytes(dev["prefix"], dev["priv"], (S, R, Hq, D), off),
                         dtype=torch.uint8, device=G.DEV)
        want = torch.empty((S, R, Hq, D), dtype=torch.bfloat16, device=G.DEV)
        got = torch.full_like(want, 7.0)
        args = (dev["prefix"], lens, dev["priv"], priv_len, dev["q"], dev["k"], dev["v"], off, mask, scale)
        B.bc_attn_step(*args, want, ws)
        B.bc_attn_step_static(*args, got)
        torch.cuda.synchronize()
        assert torch.equal(got, want), "static entry differs from the workspace entry"
        ref = OA.attention_step(host["q"], host["pk"], host["pv"], lens, host["k"], host["v"], off,
                                OA.MASK_BIDIR if mask == B.BC_MASK_BLOCK_BIDIR else OA.MASK_CAUSAL, scale=scale,
                                priv_k=host["vk"], priv_v=host["vv"], priv_len=priv_len)
        err = np.abs(got.float().cpu().numpy() - ref).max()
        assert err <= 1e-2, "static entry: max-abs %.3g against the oracle" % err


def test_static_entry_refuses_what_the_scratch_cannot_hold():
    # 64 rollouts x 64 rows x 16 heads: even one prefix split needs two
    # compact records of 272 bytes per output row, 35.7 MB > 32 MiB
    S, R, Hq, Hkv, D = 64, 64, 16, 2, 128
    prefix = B.KVCache(torch.zeros((1, Hkv, 128, D), dtype=torch.bfloat16, device=G.DEV),
                       torch.zeros((1, Hkv, 128, D), dtype=torch.bfloat16, device=G.DEV))
    priv = B.KVCache(torch.zeros((S, Hkv, 1, D), dtype=torch.bfloat16, device=G.DEV),
                     torch.zeros((S, Hkv, 1, D), dtype=torch.bfloat16, device=G.DEV))
    q = torch.zeros((S, R, Hq, D), dtype=torch.bfloat16, device=G.DEV)
    kv = torch.zeros((S, Hkv, R, D), dtype=torch.bfloat16, device=G.DEV)
    out = torch.full_like(q, 3.0)
    assert B.bc_attn_workspace_bytes(prefix, priv, (S, R, Hq, D), [0, R], 1) > B.BC_STATIC_SCRATCH_BYTES
    st = B.bc_attn_step_static(prefix, [128], priv, [0] * S, q, kv, kv, [0, R], B.BC_MASK_BLOCK_BIDIR, 0.1, out,
                               check=False)
    assert st == B.BC_ERR_SCRATCH
    # an explicit split count the scratch cannot hold, on a shape that fits
    priv4 = B.KVCache(priv.k[:4], priv.v[:4])
    st = B.bc_attn_step_static(prefix, [128], priv4, [0] * 4, q[:4], kv[:4], kv[:4], [0, R], B.BC_MASK_BLOCK_BIDIR,
                               0.1, out, n_prefix_splits=256, check=False)
    assert B.bc_attn_workspace_bytes(prefix, priv4, (4, R, Hq, D), [0, R], 256) > B.BC_STATIC_SCRATCH_BYTES
    assert st == B.BC_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()), "a refused call wrote its output"
