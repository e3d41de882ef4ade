"""Pins of the Section Diffusion schedule oracle (Fast-dDrive method summary,
sec. 3.1 - 3.2): with section units the cached decode equals a cache-free
full recompute in which every row sees exactly the rows of its own and of
earlier sections; a later block of the same section is visible, while block
units hide it; scaffold rows are never counted, predicted or changed."""

import numpy as np
import pytest

from oracle import attention as OA, section as OS


def _inputs(seed, blocks, units, Hq, Hkv, D, V, peaks=None):
    """Seeded float32 model outputs for every (block, step): Q/K/V over the
    rows of the block's unit, logits over the block's rows."""
    unit_of = {b: u for u in units for b in u}
    cache = {}

    def f(b, st):
        if (b, st) not in cache:
            g = np.random.default_rng([seed, b, st])
            ur = sum(blocks[x] for x in unit_of[b])
            q = g.standard_normal((1, ur, Hq, D)).astype(np.float32)
            k = g.standard_normal((1, Hkv, ur, D)).astype(np.float32)
            v = g.standard_normal((1, Hkv, ur, D)).astype(np.float32)
            lg = (3.0 * g.standard_normal((blocks[b], V))).astype(np.float32)
            if peaks is not None:
                for r, t in peaks.get(b, []):
                    lg[r, t] += 40.0
            cache[(b, st)] = (q, k, v, lg)
        return cache[(b, st)]
    return f


@pytest.mark.parametrize("units", [[[0, 1], [2]], [[0], [1, 2]], [[0, 1, 2]]])
def test_section_units_equal_full_recompute(units):
    Hq, Hkv, D, V, P, steps = 4, 2, 8, 16, 5, 2
    blocks = [3, 2, 4]
    g = np.random.default_rng(7)
    pk = g.standard_normal((Hkv, P, D)).astype(np.float32)
    pv = g.standard_normal((Hkv, P, D)).astype(np.float32)
    inp = _inputs(1, blocks, units, Hq, Hkv, D, V)
    keep = {(b, st) for b in range(3) for st in range(steps)}
    n = sum(blocks)
    res = OS.section_decode(pk, pv, P, units, blocks, inp, steps, 0.9, np.ones(n, np.uint8),
                            np.full(n, -1, np.int32), keep=keep)
    # the cache holds the prefix, then each unit's last-step K/V in order
    done_k, done_v, ids = [pk], [pv], [np.zeros(P, int)]
    for ui, unit in enumerate(units):
        ur = sum(blocks[b] for b in unit)
        for b in unit:
            for st in range(steps):
                q, k, v, _ = inp(b, st)
                kk = np.concatenate(done_k + [k[0]], axis=1)          # [Hkv][N][D]
                vv = np.concatenate(done_v + [v[0]], axis=1)
                blk = np.concatenate(ids + [np.full(ur, ui + 1)])
                N = kk.shape[1]
                qq = np.zeros((N, Hq, D), np.float32)
                qq[N - ur:] = q[0]
                full = OA.full_sequence_attention(qq, kk.transpose(1, 0, 2), vv.transpose(1, 0, 2), blk,
                                                  OA.MASK_BIDIR)
                assert np.allclose(res["attention"][(b, st)][0], full[N - ur:], rtol=0, atol=1e-12)
        _, k, v, _ = inp(unit[-1], steps - 1)
        done_k.append(k[0])
        done_v.append(v[0])
        ids.append(np.full(ur, ui + 1))
    assert np.array_equal(res["cache_k"], np.concatenate(done_k, axis=1))
    assert np.array_equal(res["cache_v"], np.concatenate(done_v, axis=1))


def test_later_block_of_the_section_is_visible_only_with_section_units():
    # row 0 of block 0 aims at one key of block 1 with a logit of 60 above
    # every other: it copies that key's value when block 1 is in its unit and
    # cannot see it when units are blocks
    Hq, Hkv, D, V, P = 1, 1, 4, 8, 3
    blocks = [2, 2]
    pk = np.zeros((Hkv, P, D), np.float32)
    pv = np.ones((Hkv, P, D), np.float32)

    def make(units):
        unit_of = {b: u for u in units for b in u}

        def f(b, st):
            ur = sum(blocks[x] for x in unit_of[b])
            q = np.zeros((1, ur, Hq, D), np.float32)
            k = np.zeros((1, Hkv, ur, D), np.float32)
            v = np.zeros((1, Hkv, ur, D), np.float32)
            q[0, 0, 0, 0] = 60.0 * 2.0                      # scale 1/sqrt(4) = 1/2
            if ur == 4:
                k[0, 0, 3, 0] = 1.0                          # row 3 = block 1's second row
                v[0, 0, 3] = [5.0, -3.0, 2.0, 7.0]
            return q, k, v, np.zeros((blocks[b], V), np.float32)
        return f

    n = sum(blocks)
    sec = OS.section_decode(pk, pv, P, [[0, 1]], blocks, make([[0, 1]]), 1, 0.9, np.ones(n, np.uint8),
                            np.full(n, -1, np.int32), keep={(0, 0)})
    got = sec["attention"][(0, 0)][0, 0, 0]
    # the four other keys carry weight e^-60 each (about 1e-26)
    assert np.allclose(got, [5.0, -3.0, 2.0, 7.0], rtol=0, atol=1e-20)
    blk = OS.section_decode(pk, pv, P, [[0], [1]], blocks, make([[0], [1]]), 1, 0.9, np.ones(n, np.uint8),
                            np.full(n, -1, np.int32), keep={(0, 0)})
    # block 0's own two keys are zero, the prefix keys zero: a uniform mean
    # of the three prefix values (1) and the block's two zero values
    assert np.allclose(blk["attention"][(0, 0)][0, 0, 0], 3.0 / 5.0, atol=1e-15)


def test_scaffold_rows_are_not_counted_predicted_or_changed():
    # threshold 1: nothing "exceeds" it, so every reveal is the fallback and
    # the per-step counts follow the editable rows alone; the scaffold rows
    # carry the most confident logits of their blocks and keep their tokens
    Hq, Hkv, D, V, P, steps = 2, 1, 4, 32, 2, 8
    blocks = [40, 15, 9]                  # 32 / 12 / 6 editable rows
    kinds = []
    for size, ne in zip(blocks, (32, 12, 6)):
        k = np.zeros(size, np.uint8)
        k[np.random.default_rng(size).permutation(size)[:ne]] = 1
        kinds.append(k)
    editable = np.concatenate(kinds)
    peaks = {b: [(int(r), 3) for r in np.flatnonzero(kinds[b] == 0)] for b in range(3)}
    units = [[0], [1], [2]]
    inp = _inputs(3, blocks, units, Hq, Hkv, D, V, peaks=peaks)
    template = np.where(editable == 0, 1000 + np.arange(len(editable)), -1).astype(np.int32)
    g = np.random.default_rng(0)
    res = OS.section_decode(g.standard_normal((Hkv, P, D)), g.standard_normal((Hkv, P, D)), P, units, blocks,
                            inp, steps, 1.0, editable, template)
    assert res["n_commit"][0] == [4] * 8
    assert res["n_commit"][1] == [2, 2, 2, 2, 1, 1, 1, 1]
    assert res["n_commit"][2] == [1, 1, 1, 1, 1, 1, 0, 0]
    assert not res["masked"].any()
    sc = editable == 0
    assert np.array_equal(res["tokens"][sc], template[sc])
    assert (res["tokens"][~sc] >= 0).all()
