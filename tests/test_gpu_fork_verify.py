"""A whole fork / speculative-verify round on the GPU, every step checked
against the float64 oracle on the same seeded inputs (Fast-dDrive method
summary sec. 3.2 - 3.3): bidirectional draft pass over the shared prefix and
private blocks, threshold-0 draft argmax, causal verify pass, verify."""

import numpy as np
import pytest

from oracle import attention as OA, unmask as OU, verify as OV
from tests import gpu_util as G
from block_causal_attention_gqa_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    G.require_lib()


@pytest.mark.parametrize("N,block,temperature", [(4, 0, None), (4, 1, None), (16, 2, None), (4, 2, 0.7)])
def test_fork_verify_round_matches_oracle(N, block, temperature):
    import torch
    from block_causal_attention_gqa_amd import decode
    print("fork/verify round N=%d block=%d T=%s" % (N, block, temperature), flush=True)
    fv = decode.ForkVerify(N, seed=5, device=G.DEV, block=block, temperature=temperature)
    h = fv.host_inputs(seed=5, block=block)
    R = fv.R
    for pass_id, mode in ((0, OA.MASK_BIDIR), (1, OA.MASK_CAUSAL)):
        fv.attention(pass_id)
        torch.cuda.synchronize()
        q, k, v = h["qkv"][pass_id]
        want = OA.attention_step(q, h["pk"], h["pv"], [fv.prefix], k, v, [0, R], mode, scale=fv.scale,
                                 priv_k=h["vk"], priv_v=h["vv"], priv_len=fv.priv_len)
        got = fv.out.float().cpu().numpy()
        assert np.abs(got - want).max() <= 1e-2, "pass %d" % pass_id
    fv.draft_argmax()
    torch.cuda.synchronize()
    # the scaffold rows start revealed with the template (the same for every
    # rollout); the draft reveals exactly the editable rows
    masked0 = (1 - h["fixed"]).reshape(-1).astype(np.uint8)
    tok0 = h["tokens0"]
    assert (h["fixed"] == h["fixed"][0]).all() and 0 < h["fixed"].sum() < N * R
    m_want, t_want, n_want, _ = OU.unmask_select(h["draft_logits"], fv.blk_rows, [OU.MODE_SEMI] * N, [1] * N,
                                                 np.float32(0.0), masked0, tok0)
    assert np.array_equal(fv.masked.cpu().numpy(), m_want) and not m_want.any()
    assert np.array_equal(n_want, masked0.reshape(N, R).sum(axis=1))
    assert np.array_equal(fv.tokens.cpu().numpy(), t_want)
    assert np.array_equal(fv.n_commit.cpu().numpy(), n_want)
    fv.verify()
    torch.cuda.synchronize()
    if temperature is None:
        acc, bon = OV.spec_verify(h["verify_logits"], t_want.reshape(N, R), h["fixed"], np.zeros(N, np.int32))
    else:
        acc, bon = OV.spec_verify_sampled(h["verify_logits"], h["noise"], 1.0 / temperature, t_want.reshape(N, R),
                                          h["fixed"], np.zeros(N, np.int32))
    assert np.array_equal(fv.accept_len.cpu().numpy(), acc)
    assert np.array_equal(fv.bonus.cpu().numpy(), bon)
