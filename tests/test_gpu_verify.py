"""GPU parity of bc_spec_verify against the oracle: accept lengths and bonus
tokens bit for bit."""

import ctypes

import numpy as np
import pytest
import torch

from oracle import verify as OV
from tests import gpu_util as G
from block_causal_attention_gqa_amd import binding as B
from block_causal_attention_gqa_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    G.require_lib()


def run(logits, draft, fixed, first):
    S, L, V = logits.shape
    acc = torch.full((S,), -7, dtype=torch.int32, device=G.DEV)
    bon = torch.full((S,), -7, dtype=torch.int32, device=G.DEV)
    ws = torch.zeros(B.bc_verify_workspace_bytes(S, L, V), dtype=torch.uint8, device=G.DEV)
    B.bc_spec_verify(G.to_dev(logits), G.to_dev(draft.astype(np.int32)),
                     None if fixed is None else G.to_dev(fixed.astype(np.uint8)),
                     G.to_dev(np.asarray(first, np.int32)), acc, bon, ws)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), bon.cpu().numpy()


def compare(logits, draft, fixed, first):
    print("verify case S=%d L=%d V=%d m=%d" % (logits.shape + (draft.shape[1],)), flush=True)
    ga, gb = run(logits, draft, fixed, first)
    oa, ob = OV.spec_verify(logits, draft, fixed, first)
    assert np.array_equal(ga, oa) and np.array_equal(gb, ob)
    return ga, gb


@pytest.mark.parametrize("p_agree", [0.5, 0.8, 1.0])
@pytest.mark.parametrize("N", [1, 4])
def test_trajectory_block_agreement(p_agree, N):
    # [24 x 151936] per rollout; drafts agree with the AR argmax at rate p
    L, V = 24, 151936
    lg = np.empty((N, L, V), np.float32)
    draft = np.empty((N, L), np.int32)
    for s in range(N):
        lg[s], t = synth.argmax_planted_logits(9, L, V, 4.0, 0.5, s)
        draft[s] = synth.drafts_with_agreement(9, t, p_agree, V, s, int(p_agree * 10))
    fixed = (np.random.default_rng(N).random((N, L)) < 0.15).astype(np.uint8)
    first = np.random.default_rng(N + 1).integers(0, 5, N)
    compare(lg, draft, None, np.zeros(N, np.int32))
    compare(lg, draft, fixed, first)


def test_partial_block_and_bonus_row():
    # block of 23 drafts verified against 24 logit rows: full agreement gives
    # the bonus from row 23; m == n_lrows gives none
    V = 5000
    lg, t = synth.argmax_planted_logits(10, 24, V, 4.0, 1.0, 0)
    compare(lg[None], t[None, :23].copy(), None, [0])
    compare(lg[None], t[None].copy(), None, [0])
    compare(lg[None], t[None].copy(), None, [24])
    compare(lg[None], t[None, :23].copy(), None, [23])


def test_ties_take_lowest_index():
    lg = np.zeros((1, 3, 300), np.float32)
    lg[0, 0, [7, 200]] = 1.0
    lg[0, 1, [250, 13]] = 2.0
    lg[0, 2, :] = -1.0
    compare(lg, np.array([[7, 13, 0]], np.int32), None, [0])
    compare(lg, np.array([[200, 13, 0]], np.int32), None, [0])


@pytest.mark.parametrize("V", [1, 7, 8191, 8193])
def test_odd_vocab(V):
    rng = np.random.default_rng(V)
    lg = rng.standard_normal((3, 6, V)).astype(np.float32)
    draft = rng.integers(0, V, (3, 5)).astype(np.int32)
    compare(lg, draft, None, [0, 2, 5])


def test_argument_errors():
    lg = G.to_dev(np.zeros((1, 4, 10), np.float32))
    d = G.to_dev(np.zeros((1, 5), np.int32))
    f = G.to_dev(np.zeros(1, np.int32))
    a = torch.zeros(1, dtype=torch.int32, device=G.DEV)
    ws = torch.zeros(4096, dtype=torch.uint8, device=G.DEV)
    assert B.bc_spec_verify(lg, d, None, f, a, a.clone(), ws, check=False) == B.BC_ERR_ARG  # m > n_lrows


@pytest.mark.parametrize("inv_t", [1.0, 1.0 / 0.7, 2.0])
@pytest.mark.parametrize("V", [151936, 1001])
def test_sampled_verify_matches_oracle(inv_t, V):
    # trajectory-only sampling: Gumbel-max over supplied noise, drafts taken
    # from the oracle's sampled tokens with 80% agreement
    S, L, m = 4, 24, 24
    print("sampled verify V=%d inv_t=%.3f" % (V, inv_t), flush=True)
    x = synth.logits(70, S * L, V, 4.0, 0).reshape(S, L, V)
    g = synth.gumbel(70, (S, L, V), 0)
    t = np.array([[OV.argmax_lowest(OV.perturbed_row(x[s, i], g[s, i], inv_t)) for i in range(L)]
                  for s in range(S)], np.int32)
    draft = np.stack([synth.drafts_with_agreement(70, t[s, :m], 0.8, V, s) for s in range(S)])
    fixed = (np.random.default_rng(70).random((S, m)) < 0.3).astype(np.uint8)
    first = np.array([0, 3, 10, 24], np.int32)
    acc = torch.full((S,), -7, dtype=torch.int32, device=G.DEV)
    bon = torch.full((S,), -7, dtype=torch.int32, device=G.DEV)
    ws = torch.zeros(B.bc_verify_workspace_bytes(S, L, V), dtype=torch.uint8, device=G.DEV)
    B.bc_spec_verify_sampled(G.to_dev(x), G.to_dev(g), inv_t, G.to_dev(draft), G.to_dev(fixed), G.to_dev(first),
                             acc, bon, ws)
    torch.cuda.synchronize()
    oa, ob = OV.spec_verify_sampled(x, g, inv_t, draft, fixed, first)
    assert np.array_equal(acc.cpu().numpy(), oa)
    assert np.array_equal(bon.cpu().numpy(), ob)


def test_sampled_verify_argument_errors():
    S, L, V = 1, 4, 64
    x = G.to_dev(np.zeros((S, L, V), np.float32))
    d = G.to_dev(np.zeros((S, L), np.int32))
    f = G.to_dev(np.zeros(S, np.int32))
    acc = torch.zeros(S, dtype=torch.int32, device=G.DEV)
    bon = torch.zeros(S, dtype=torch.int32, device=G.DEV)
    ws = torch.zeros(B.bc_verify_workspace_bytes(S, L, V), dtype=torch.uint8, device=G.DEV)
    for inv_t in (0.0, -1.0, float("nan"), float("inf")):
        assert B.bc_spec_verify_sampled(x, x, inv_t, d, None, f, acc, bon, ws, check=False) == B.BC_ERR_ARG
    st = B.lib().bc_spec_verify_sampled(x.data_ptr(), None, ctypes.c_float(1.0), S, L, V, d.data_ptr(), L, None,
                                        f.data_ptr(), acc.data_ptr(), bon.data_ptr(), ws.data_ptr(), ws.numel(), None)
    assert st == B.BC_ERR_ARG


@pytest.mark.parametrize("S,L", [(64, 64), (1, 4096)])
def test_scan_row_limit(S, L):
    # S * L = 4096 logit rows, the most one call takes: 64 rollouts of 64 rows,
    # and one sequence of 4096
    assert S * L == B.BC_MAX_SCAN_ROWS
    V = 2048
    lg = np.empty((S, L, V), np.float32)
    draft = np.empty((S, L), np.int32)
    for s in range(S):
        lg[s], t = synth.argmax_planted_logits(12, L, V, 4.0, 0.5, s)
        draft[s] = synth.drafts_with_agreement(12, t, 0.97 if S > 1 else 0.999, V, s)
    fixed = (np.random.default_rng(S).random((S, L)) < 0.1).astype(np.uint8)
    first = np.random.default_rng(S + 1).integers(0, 8, S)
    compare(lg, draft, None, np.zeros(S, np.int32))
    compare(lg, draft, fixed, first)


def test_one_past_the_scan_row_limit_is_unsupported():
    S, L, V = 65, 64, 4
    lg = G.to_dev(np.zeros((S, L, V), np.float32))
    d = G.to_dev(np.zeros((S, L), np.int32))
    f = G.to_dev(np.zeros(S, np.int32))
    a = torch.zeros(S, dtype=torch.int32, device=G.DEV)
    ws = torch.zeros(B.bc_verify_workspace_bytes(64, L, V), dtype=torch.uint8, device=G.DEV)
    assert B.bc_verify_workspace_bytes(S, L, V) == 0
    assert B.bc_spec_verify(lg, d, None, f, a, a.clone(), ws, check=False) == B.BC_ERR_UNSUPPORTED


def test_vocabulary_past_one_merge_round():
    # more than 64 chunks of 4096 logits: two merge rounds per row; four
    # correct drafts over five rows, so the bonus is row 4's argmax, planted
    # in the last chunk
    V = 64 * 4096 + 4097
    lg, _ = synth.argmax_planted_logits(13, 5, V, 4.0, 0.5, 0)
    lg[4, V - 2] = lg[4].max() + 1.0
    t = lg.argmax(axis=1).astype(np.int32)
    ga, gb = compare(lg[None], t[None, :4].copy(), None, [0])
    assert ga[0] == 4 and gb[0] == V - 2
