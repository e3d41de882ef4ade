"""GPU parity of bc_unmask_select against the float64 oracle: the revealed
set, tokens and per-block counts must match bit for bit; the float32
confidence output is compared with a relative tolerance."""

import math

import numpy as np
import pytest
import torch

from oracle import unmask as OU
from tests import gpu_util as G
from block_causal_attention_gqa_amd import binding as B
from block_causal_attention_gqa_amd import synth

pytestmark = pytest.mark.gpu
SEMI, FULL = B.BC_UNMASK_SEMI, B.BC_UNMASK_FULL
NEG = np.float32(-1e30)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    G.require_lib()


def run_gpu(logits, blk_off, mode, n_div, tau, masked, tokens):
    R, V = logits.shape
    lg = G.to_dev(logits)
    m = G.to_dev(masked.astype(np.uint8))
    t = G.to_dev(tokens.astype(np.int32))
    conf = torch.full((R,), float("nan"), dtype=torch.float32, device=G.DEV)
    nc = torch.full((len(blk_off) - 1,), -7, dtype=torch.int32, device=G.DEV)
    ws = torch.zeros(B.bc_unmask_workspace_bytes(R, V), dtype=torch.uint8, device=G.DEV)
    B.bc_unmask_select(lg, blk_off, mode, n_div, tau, m, t, conf, nc, ws)
    torch.cuda.synchronize()
    return m.cpu().numpy(), t.cpu().numpy(), nc.cpu().numpy(), conf.cpu().numpy()


def compare(logits, blk_off, mode, n_div, tau, masked, tokens):
    print("unmask case R=%d V=%d blk=%s mode=%s n_div=%s" % (logits.shape[0], logits.shape[1],
          list(blk_off)[:5], list(mode)[:4], list(n_div)[:4]), flush=True)
    gm, gt, gn, gc = run_gpu(logits, blk_off, mode, n_div, tau, masked, tokens)
    om, ot, on, oc = OU.unmask_select(logits, blk_off, mode, n_div, np.float32(tau), masked, tokens)
    assert np.array_equal(gm, om), "revealed set differs"
    assert np.array_equal(gt, ot), "tokens differ"
    assert np.array_equal(gn, on), "commit counts differ"
    sel = masked.astype(bool)
    np.testing.assert_allclose(gc[sel], oc[sel], rtol=2e-5, atol=0)
    return gm, gt


def test_tiny_config():
    # [8 x 1024] ~ N(0, 3^2), threshold 0.9, at least one reveal per step
    x = synth.logits(0, 8, 1024, 3.0, 0)
    compare(x, [0, 8], [FULL], [1 << 30], 0.9, np.ones(8, np.uint8), np.full(8, -1, np.int32))


def test_tiny_config_runs_until_complete():
    masked = np.ones(8, np.uint8)
    tokens = np.full(8, -1, np.int32)
    for step in range(8):
        x = synth.logits(0, 8, 1024, 3.0, step)
        synth.plant_peaks(x, 0, 0.2, 9.0, step)
        masked, tokens = compare(x, [0, 8], [FULL], [1 << 30], 0.9, masked, tokens)
        if masked.sum() == 0:
            break
    assert masked.sum() == 0


@pytest.mark.parametrize("bs", [32, 12, 6])
def test_section_block_schedule(bs):
    # full vocabulary 151936, sigma 4, 8 steps with n = steps left
    masked = np.ones(bs, np.uint8)
    tokens = np.full(bs, -1, np.int32)
    for step in range(8):
        x = synth.logits(3, bs, 151936, 4.0, bs, step)
        synth.plant_peaks(x, 3, 0.1, 12.0, bs, step)
        masked, tokens = compare(x, [0, bs], [FULL], [8 - step], 0.9, masked, tokens)
    assert masked.sum() == 0


def test_pipelined_semi_and_full_blocks():
    rng = np.random.default_rng(4)
    x = synth.logits(4, 21, 2048, 4.0, 0)
    synth.plant_peaks(x, 4, 0.3, 10.0, 0)
    masked = np.ones(21, np.uint8)
    # completion ratios -> committed rows, seeded
    for b in range(3):
        r = rng.random()
        done = rng.choice(7, size=int(r * 7), replace=False)
        masked[7 * b + done] = 0
    compare(x, [0, 7, 14, 21], [FULL, SEMI, SEMI], [1 << 30, 1, 1], 0.9, masked, np.full(21, -1, np.int32))


def _two_value(a, V):
    row = np.full(V, NEG, np.float32)
    row[0] = np.float32(a)
    row[1] = 0.0
    return row


def test_threshold_band_rows_are_decided_in_float64():
    # confidences within 1e-9 of the threshold: inside the float32 error band,
    # so the kernel must recompute them in float64 to agree with the oracle
    V = 4096
    t = float(np.float32(0.9))
    rows = []
    for c in [t + 1e-9, t - 1e-9, t + 3e-9, t - 3e-9, t + 2e-8, t - 2e-8, 0.3, 0.95]:
        a = math.log(c / (1 - c))
        rows.append(_two_value(a, V))
    x = np.stack(rows)
    for mode in (SEMI, FULL):
        compare(x, [0, 8], [mode], [4], 0.9, np.ones(8, np.uint8), np.zeros(8, np.int32))


def test_rank_cut_near_ties_and_exact_ties():
    V = 4096
    gaps = [0.5, 0.5 + 1e-7, 0.5 - 1e-7, 0.5, 0.1, 0.7, 0.5 + 2e-7, 0.3]
    x = np.stack([_two_value(a, V) for a in gaps])
    x[3] = x[0]                       # exact duplicate rows: lower index wins
    for n in (1, 2, 3, 4, 8):
        compare(x, [0, 8], [FULL], [n], 0.9, np.ones(8, np.uint8), np.zeros(8, np.int32))


def test_float32_tied_confidences_around_the_cut():
    # two-value rows with logits a and the next float32 above it, a ~ 1e-3:
    # their confidences differ in float64 (by ~1e-10 relative) but round to
    # one float32, and the larger sits at the higher row, so float32 order
    # with the row tie-break disagrees with float64 order.  Sweeping n moves
    # the rank cut onto, beside and away from the tied pairs; decisions must
    # match the float64 oracle in every case.
    V = 4096
    base = [np.float32(1e-3), np.float32(2e-3), np.float32(0.2), np.float32(5e-4)]
    a = []
    for v in base:
        a += [v, np.nextafter(v, np.float32(1.0))]        # lower logit first
    x = np.stack([_two_value(float(v), V) for v in a])
    conf = [1.0 / (1.0 + math.exp(-float(v))) for v in a]     # two finite logits: a and 0
    for j in range(0, 8, 2):
        assert conf[j] != conf[j + 1] and np.float32(conf[j]) == np.float32(conf[j + 1])
    for n in range(1, 9):
        compare(x, [0, 8], [FULL], [n], 0.9, np.ones(8, np.uint8), np.zeros(8, np.int32))
    # the same rows in a block of 40 with random others around them
    y = np.concatenate([x, synth.logits(8, 32, V, 4.0, 0)])
    for n in (3, 5, 8, 13):
        compare(y, [0, 40], [FULL], [n], 0.9, np.ones(40, np.uint8), np.zeros(40, np.int32))


def test_argmax_ties_and_uniform_rows():
    V = 1000
    x = np.zeros((4, V), np.float32)
    x[1, [5, 900]] = 3.0
    x[2, [999, 998]] = 1.0
    x[3] = synth.logits(5, 1, V, 1.0, 0)[0]
    compare(x, [0, 4], [FULL], [1], 0.9, np.ones(4, np.uint8), np.zeros(4, np.int32))


@pytest.mark.parametrize("V", [1, 3, 1023, 8193, 70001])
def test_odd_vocab_sizes(V):
    x = synth.logits(6, 5, V, 4.0, V)
    compare(x, [0, 2, 5], [FULL, FULL], [2, 1], 0.9, np.ones(5, np.uint8), np.zeros(5, np.int32))


def test_many_blocks_batch():
    # 16 sequences' blocks of 32 in one call (large-block decode at batch 16)
    R, V = 16 * 32, 151936
    x = synth.logits(7, R, V, 4.0, 0)
    synth.plant_peaks(x, 7, 0.05, 12.0, 0)
    masked = (np.random.default_rng(7).random(R) < 0.7).astype(np.uint8)
    compare(x, list(range(0, R + 1, 32)), [FULL] * 16, [3] * 16, 0.9, masked, np.zeros(R, np.int32))


def test_nothing_masked_and_errors():
    x = synth.logits(8, 4, 64, 4.0, 0)
    gm, gt, gn, _ = run_gpu(x, [0, 4], [FULL], [1], 0.9, np.zeros(4, np.uint8), np.arange(4, dtype=np.int32))
    assert gm.sum() == 0 and list(gt) == [0, 1, 2, 3] and gn[0] == 0
    lg = G.to_dev(x)
    m = G.to_dev(np.ones(4, np.uint8))
    t = G.to_dev(np.zeros(4, np.int32))
    nc = torch.zeros(1, dtype=torch.int32, device=G.DEV)
    ws = torch.zeros(B.bc_unmask_workspace_bytes(4, 64), dtype=torch.uint8, device=G.DEV)
    assert B.bc_unmask_select(lg, [0, 4], [FULL], [0], 0.9, m, t, None, nc, ws, check=False) == B.BC_ERR_ARG
    assert B.bc_unmask_select(lg, [0, 3], [FULL], [1], 0.9, m, t, None, nc, ws, check=False) == B.BC_ERR_ARG
    assert B.bc_unmask_select(lg, [0, 4], [2], [1], 0.9, m, t, None, nc, ws, check=False) == B.BC_ERR_ARG
    assert B.bc_unmask_select(lg, [0, 4], [FULL], [1], 0.9, m, t, None, nc, ws[:8], check=False) \
        == B.BC_ERR_WORKSPACE


def test_block_with_nothing_masked_reports_zero():
    # the middle block has no masked rows: its count must still be written
    x = synth.logits(9, 12, 3000, 4.0, 0)
    masked = np.array([1, 0, 1, 1, 0, 0, 0, 0, 1, 1, 1, 1], np.uint8)
    compare(x, [0, 4, 8, 12], [FULL, FULL, SEMI], [2, 1, 1], 0.9, masked, np.zeros(12, np.int32))


def test_one_workspace_across_shapes_and_entry_points():
    # a workspace zeroed once serves calls of different row counts and vocab
    # sizes, and a verify call, in any order (the counters sit at a fixed
    # place and every call leaves them at zero)
    from oracle import verify as OV
    ws = torch.zeros(B.bc_unmask_workspace_bytes(64, 151936), dtype=torch.uint8, device=G.DEV)
    rng = np.random.default_rng(21)
    for it, (R, V) in enumerate([(12, 151936), (32, 151936), (6, 151936), (64, 5000), (32, 151936),
                                 (7, 3001), (32, 151936)]):
        x = synth.logits(21, R, V, 4.0, it)
        masked = (rng.random(R) < 0.8).astype(np.uint8)
        m = G.to_dev(masked)
        t = G.to_dev(np.zeros(R, np.int32))
        nc = torch.full((2,), -7, dtype=torch.int32, device=G.DEV)
        half = R // 2
        B.bc_unmask_select(G.to_dev(x), [0, half, R], [FULL, FULL], [3, 2], 0.9, m, t, None, nc, ws)
        om, ot, on, _ = OU.unmask_select(x, [0, half, R], [FULL, FULL], [3, 2], np.float32(0.9),
                                         masked, np.zeros(R, np.int32))
        assert np.array_equal(m.cpu().numpy(), om) and np.array_equal(t.cpu().numpy(), ot)
        assert np.array_equal(nc.cpu().numpy(), on)
        if it % 2 == 1:
            lg, tg = synth.argmax_planted_logits(21, 24, 151936, 4.0, 0.5, it)
            d = synth.drafts_with_agreement(21, tg[:23], 0.8, 151936, it)
            acc = torch.full((1,), -7, dtype=torch.int32, device=G.DEV)
            bon = torch.full((1,), -7, dtype=torch.int32, device=G.DEV)
            B.bc_spec_verify(G.to_dev(lg[None]), G.to_dev(d[None]), None,
                             G.to_dev(np.zeros(1, np.int32)), acc, bon, ws)
            oa, ob = OV.spec_verify(lg[None], d[None], None, [0])
            assert int(acc.item()) == int(oa[0]) and int(bon.item()) == int(ob[0])


def test_scan_then_decide_equals_select():
    R, V = 40, 151936
    x = synth.logits(30, R, V, 4.0, 0)
    synth.plant_peaks(x, 30, 0.2, 12.0, 0)
    lg = G.to_dev(x)
    masked0 = (np.random.default_rng(30).random(R) < 0.75).astype(np.uint8)
    outs = []
    for split in (False, True):
        m = G.to_dev(masked0)
        t = G.to_dev(np.full(R, -1, np.int32))
        c = torch.full((R,), float("nan"), dtype=torch.float32, device=G.DEV)
        nc = torch.full((2,), -7, dtype=torch.int32, device=G.DEV)
        ws = torch.empty(B.bc_unmask_workspace_bytes(R, V), dtype=torch.uint8, device=G.DEV)
        args = (lg, [0, 16, R], [FULL, SEMI], [3, 1], 0.9, m, t, c, nc, ws)
        if split:
            B.bc_vocab_scan(lg, m, True, ws)
            B.bc_unmask_decide(*args)
        else:
            B.bc_unmask_select(*args)
        torch.cuda.synchronize()
        outs.append([z.cpu().numpy() for z in (m, t, c, nc)])
    for u, w in zip(*outs):
        assert np.array_equal(u, w, equal_nan=True) if u.dtype.kind == "f" else np.array_equal(u, w)


@pytest.mark.parametrize("sizes", [[64], [65], [200, 64, 1], [63, 2, 129]])
def test_block_sizes_around_one_wave(sizes):
    # blocks of up to 64 rows are decided by one wave, larger ones by the
    # whole workgroup; both must agree with the oracle, with confident rows
    # planted so that both the threshold and the ranking branches run
    R, V = sum(sizes), 3000
    x = synth.logits(80 + len(sizes), R, V, 4.0, 0)
    synth.plant_peaks(x, 80 + len(sizes), 0.25, 12.0, 0)
    off = np.concatenate([[0], np.cumsum(sizes)]).tolist()
    masked = (np.random.default_rng(80 + R).random(R) < 0.8).astype(np.uint8)
    nb = len(sizes)
    compare(x, off, [FULL, SEMI, FULL, FULL][:nb], [5, 1, 3, 2][:nb], 0.9, masked, np.zeros(R, np.int32))


# ---- the call limits: BC_MAX_SCAN_ROWS rows, BC_MAX_BLOCKS blocks,
# BC_MAX_BLOCK_ROWS rows in one block, and one past each


def test_max_scan_rows_in_max_blocks():
    # 4096 rows in 64 blocks of 64: alternating modes, divisors 1..8, blocks
    # fully masked, half masked and not masked at all
    nb, bs, V = B.BC_MAX_BLOCKS, 64, 4096
    R = nb * bs
    assert R == B.BC_MAX_SCAN_ROWS
    x = synth.logits(90, R, V, 4.0, 0)
    synth.plant_peaks(x, 90, 0.15, 12.0, 0)
    rng = np.random.default_rng(90)
    frac = rng.choice([0.0, 0.5, 1.0], nb)
    masked = (rng.random(R) < np.repeat(frac, bs)).astype(np.uint8)
    modes = [FULL if b % 2 else SEMI for b in range(nb)]
    divs = [1 + b % 8 for b in range(nb)]
    compare(x, list(range(0, R + 1, bs)), modes, divs, 0.9, masked, np.zeros(R, np.int32))


@pytest.mark.parametrize("n_blk", [1, 4])
def test_blocks_of_max_rows(n_blk):
    # blocks of 1024 rows (the workgroup decide path at its largest); four of
    # them fill the scan-row limit
    bs, V = B.BC_MAX_BLOCK_ROWS, 2048
    R = n_blk * bs
    x = synth.logits(91, R, V, 4.0, n_blk)
    synth.plant_peaks(x, 91, 0.1, 12.0, n_blk)
    masked = (np.random.default_rng(91 + n_blk).random(R) < 0.9).astype(np.uint8)
    compare(x, list(range(0, R + 1, bs)), [FULL, SEMI, FULL, FULL][:n_blk], [3, 1, 7, 1024][:n_blk], 0.9,
            masked, np.zeros(R, np.int32))


def test_one_past_each_limit_is_unsupported():
    V = 8

    def status(R, off):
        lg = G.to_dev(np.zeros((R, V), np.float32))
        m = G.to_dev(np.ones(R, np.uint8))
        t = G.to_dev(np.zeros(R, np.int32))
        nc = torch.zeros(len(off) - 1, dtype=torch.int32, device=G.DEV)
        ws = torch.zeros(B.bc_unmask_workspace_bytes(min(R, B.BC_MAX_SCAN_ROWS), V), dtype=torch.uint8,
                         device=G.DEV)
        n = len(off) - 1
        return B.bc_unmask_select(lg, off, [FULL] * n, [1] * n, 0.9, m, t, None, nc, ws, check=False)

    R = B.BC_MAX_SCAN_ROWS + 1
    assert status(R, [0, 1024, 2048, 3072, 4096, R]) == B.BC_ERR_UNSUPPORTED
    assert status(B.BC_MAX_BLOCK_ROWS + 1, [0, B.BC_MAX_BLOCK_ROWS + 1]) == B.BC_ERR_UNSUPPORTED
    nb = B.BC_MAX_BLOCKS + 1
    assert status(nb, list(range(nb + 1))) == B.BC_ERR_UNSUPPORTED
    assert B.bc_unmask_workspace_bytes(B.BC_MAX_SCAN_ROWS + 1, V) == 0
    # the limits themselves are accepted
    assert status(B.BC_MAX_BLOCK_ROWS, [0, B.BC_MAX_BLOCK_ROWS]) == B.BC_OK
    assert status(B.BC_MAX_BLOCKS, list(range(B.BC_MAX_BLOCKS + 1))) == B.BC_OK


def test_vocabulary_past_one_merge_round():
    # more than 64 chunks of 4096 logits: the decide merges each row's chunk
    # partials in two rounds of loads
    V = 64 * 4096 + 4097
    x = synth.logits(93, 6, V, 4.0, 0)
    synth.plant_peaks(x, 93, 0.5, 14.0, 0)
    x[2, V - 1] = 40.0          # argmax in the last chunk
    compare(x, [0, 3, 6], [FULL, SEMI], [2, 1], 0.9, np.ones(6, np.uint8), np.zeros(6, np.int32))


def test_permuted_rows_straddling_the_rank_cut():
    # rows whose logits are permutations of one row have equal confidences
    # by definition; the order in which a sum runs must not split them, so
    # the cut takes the lowest row indexes among them.  Rows 1, 3, 4, 6 are
    # one row permuted, 0 and 5 above them, 2 and 7 below; n sweeps the cut
    # across the tied rows.  Then the same rows spread through a block of 64
    # with random rows in between.
    rng = np.random.default_rng(31)
    for V in (4096, 151936):
        base = (rng.standard_normal(V) * 2.0).astype(np.float32)
        x = np.empty((8, V), np.float32)
        for i in (1, 3, 4, 6):
            x[i] = base[rng.permutation(V)]
        for i, peak in ((0, 9.0), (5, 8.0)):
            x[i] = rng.standard_normal(V).astype(np.float32) * 2.0
            x[i][rng.integers(V)] += np.float32(peak)
        for i in (2, 7):
            x[i] = (rng.standard_normal(V) * 0.5).astype(np.float32)
        for n in (1, 2, 3, 4):
            gm, _ = compare(x, [0, 8], [FULL], [n], 0.999, np.ones(8, np.uint8), np.zeros(8, np.int32))
        mk = np.ones(8, np.uint8)
        mk[[0, 1]] = 0
        compare(x, [0, 8], [FULL], [2], 0.999, mk, np.zeros(8, np.int32))
        y = synth.logits(9, 64, V, 1.0, V)
        at = rng.choice(64, 8, replace=False)
        y[at] = x
        for n in (13, 16, 22, 32):          # k = 5, 4, 3, 2: the tied rows rank 3rd to 6th
            compare(y, [0, 64], [FULL], [n], 0.999, np.ones(64, np.uint8), np.zeros(64, np.int32))
