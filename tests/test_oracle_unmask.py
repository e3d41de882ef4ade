"""Pins of the unmask oracle: closed-form confidences, hand-built selections,
the step-budget schedule, monotone reveals and subset brute force."""

import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import unmask as U

NEG = np.float32(-1e30)


def two_value_row(a, vocab=64):
    """[a, 0, -1e30, ...]: confidence 1 / (1 + e^-a) in closed form (a >= 0)."""
    row = np.full(vocab, NEG, dtype=np.float32)
    row[0] = np.float32(a)
    row[1] = 0.0
    return row


def test_uniform_row_confidence_is_one_over_vocab():
    for v in (1, 7, 1024, 151936):
        m, a, s, c = U.row_confidence(np.full(v, 2.5, np.float32))
        assert a == 0 and m == 2.5 and s == float(v)
        assert c == 1.0 / v


def test_two_value_row_closed_form():
    for a in (0.0, 0.5, 2.0, 2.1972246, 7.0):
        _, arg, _, c = U.row_confidence(two_value_row(a))
        a32 = float(np.float32(a))
        assert arg == 0
        assert abs(c - 1.0 / (1.0 + math.exp(-a32))) < 1e-15


def test_argmax_ties_take_lowest_index():
    row = np.zeros(10, np.float32)
    row[[3, 7]] = 5.0
    assert U.row_confidence(row)[1] == 3
    row[1] = 5.0
    assert U.row_confidence(row)[1] == 1


def _logit_a_for_conf(c):
    """logit gap a with 1 / (1 + e^-a) == c."""
    return math.log(c / (1.0 - c))


def test_semi_commits_exactly_rows_above_threshold():
    # rows with confidence just above / just below 0.9; SEMI reveals exactly
    # the ones above (strict), whatever their count
    tau = np.float32(0.9)
    t = float(tau)
    confs = [t + 1e-7, t - 1e-7, 0.5, 0.99, t - 1e-6, t + 3e-6]
    above = [0, 3, 5]
    logits = np.stack([two_value_row(_logit_a_for_conf(c)) for c in confs])
    mo, to, n, conf = U.unmask_select(logits, [0, 6], [U.MODE_SEMI], [1], tau,
                                      np.ones(6, np.uint8), np.full(6, -1, np.int32))
    assert list(np.flatnonzero(mo == 0)) == above
    assert n[0] == 3
    assert all(to[r] == 0 for r in above) and all(to[r] == -1 for r in (1, 2, 4))


def test_full_fallback_takes_the_most_confident_rows():
    # nothing above the threshold: FULL reveals ceil(|E| / n) rows, the most
    # confident ones; equal confidences go to the lower row index
    gaps = [0.1, 0.9, 0.3, 0.9, 1.5, 0.2, 1.1, 0.0]
    logits = np.stack([two_value_row(a) for a in gaps])
    masked = np.ones(8, np.uint8)
    mo, _, n, _ = U.unmask_select(logits, [0, 8], [U.MODE_FULL], [3], 0.9, masked,
                                  np.zeros(8, np.int32))
    assert n[0] == 3                               # ceil(8 / 3)
    assert sorted(np.flatnonzero(mo == 0)) == [1, 4, 6]   # 1.5, 1.1, then 0.9 @ row 1 (not 3)


def test_full_takes_all_above_threshold_when_more_than_fallback():
    gaps = [3.0, 3.1, 3.2, 0.1, 0.2, 2.5]          # conf(3.0) = 0.9526 > 0.9
    logits = np.stack([two_value_row(a) for a in gaps])
    mo, _, n, _ = U.unmask_select(logits, [0, 6], [U.MODE_FULL], [6], 0.9,
                                  np.ones(6, np.uint8), np.zeros(6, np.int32))
    assert n[0] == 4                               # 3.0 3.1 3.2 2.5 (0.924) > 0.9
    assert sorted(np.flatnonzero(mo == 0)) == [0, 1, 2, 5]


def test_step_budget_schedule_completes_block_exactly():
    # Reading of the 1/n fallback: n = steps left in a fixed budget.  32 rows
    # over 8 steps reveal 4 per step; 12 rows reveal 2,2,2,2,1,1,1,1.
    for rows, steps, want in ((32, 8, [4] * 8), (12, 8, [2, 2, 2, 2, 1, 1, 1, 1]),
                              (6, 8, [1] * 6 + [0, 0]), (32, 16, [2] * 16)):
        masked = np.ones(rows, np.uint8)
        tokens = np.full(rows, -1, np.int32)
        got = []
        for s in range(steps):
            lg = np.random.default_rng(s).standard_normal((rows, 512)).astype(np.float32)  # conf << 0.9
            masked2, tokens2, n, _ = U.unmask_select(lg, [0, rows], [U.MODE_FULL],
                                                     [steps - s], 0.9, masked, tokens)
            # monotone: nothing revealed before changes or is re-masked
            assert np.all(masked2 <= masked)
            keep = masked == 0
            assert np.array_equal(tokens2[keep], tokens[keep])
            got.append(int(n[0]))
            masked, tokens = masked2, tokens2
        assert got == want
        assert masked.sum() == 0 and np.all(tokens >= 0)


def test_unmasked_rows_are_ignored():
    logits = np.stack([two_value_row(a) for a in (9.0, 0.1, 0.2)])
    masked = np.array([0, 1, 1], np.uint8)
    tokens = np.array([17, -1, -1], np.int32)
    mo, to, n, conf = U.unmask_select(logits, [0, 3], [U.MODE_FULL], [2], 0.9, masked, tokens)
    assert to[0] == 17 and np.isnan(conf[0])
    assert n[0] == 1 and list(mo) == [0, 1, 0]      # 0.2 beats 0.1


def test_blocks_are_independent():
    gaps = [0.1, 0.2, 0.3, 4.0, 0.5, 0.6]
    logits = np.stack([two_value_row(a) for a in gaps])
    mo, _, n, _ = U.unmask_select(logits, [0, 2, 6], [U.MODE_FULL, U.MODE_SEMI], [1, 1], 0.9,
                                  np.ones(6, np.uint8), np.zeros(6, np.int32))
    assert list(n) == [2, 1]
    assert list(mo) == [0, 0, 1, 0, 1, 1]


@pytest.mark.parametrize("seed", range(6))
def test_selection_brute_force_over_subsets(seed):
    # The committed set must be the unique k-subset all of whose members come
    # before every non-member in (confidence desc, row asc) order; found here
    # by enumerating every subset of the masked rows.
    rng = np.random.default_rng(seed)
    R = 9
    gaps = rng.choice([0.0, 0.5, 1.0, 2.0, 2.5, 3.0], size=R)
    logits = np.stack([two_value_row(a) for a in gaps])
    masked = (rng.random(R) < 0.8).astype(np.uint8)
    E = [r for r in range(R) if masked[r]]
    conf = {r: 1.0 / (1.0 + math.exp(-float(np.float32(gaps[r])))) for r in E}
    for mode in (U.MODE_SEMI, U.MODE_FULL):
        n_div = int(rng.integers(1, 5))
        mo, _, n, _ = U.unmask_select(logits, [0, R], [mode], [n_div], 0.9, masked,
                                      np.zeros(R, np.int32))
        chosen = set(r for r in E if mo[r] == 0)
        k = len(chosen)
        n_above = sum(1 for r in E if conf[r] > float(np.float32(0.9)))
        want_k = n_above if mode == U.MODE_SEMI else min(len(E), max(n_above, math.ceil(len(E) / n_div)))
        assert k == want_k == n[0]

        def before(a, b):
            return conf[a] > conf[b] or (conf[a] == conf[b] and a < b)
        valid = [set(c) for c in itertools.combinations(E, k)
                 if all(before(a, b) for a in c for b in E if b not in c)]
        assert valid == [chosen]


def test_section_table_block_counts(golden_dir):
    # Fast-dDrive method summary sec. 3.2: n_s = ceil(|E_s| / d) blocks per
    # section; with d = 32 this reproduces the printed counts 1 / 6 / 1 / 3.
    with open(os.path.join(golden_dir, "section_table.json")) as f:
        table = json.load(f)
    for sec in table["sections"]:
        assert math.ceil(sec["editable"] / 32) == sec["blocks"]
    edit = sum(s["editable"] for s in table["sections"])
    scaf = sum(s["scaffold"] for s in table["sections"])
    assert edit == 280
    assert abs(scaf / (edit + scaf) - table["scaffold_fraction_approx"]) < 0.02


def test_threshold_comparison_is_strict():
    # a uniform row of 4 has confidence exactly 0.25, which is also exactly a
    # float32 threshold: "exceeds" must not reveal it
    logits = np.stack([np.zeros(4, np.float32), np.array([0.01, 0, 0, 0], np.float32)])
    mo, _, n, conf = U.unmask_select(logits, [0, 2], [U.MODE_SEMI], [1], np.float32(0.25),
                                     np.ones(2, np.uint8), np.zeros(2, np.int32))
    assert conf[0] == 0.25 and conf[1] > 0.25
    assert list(mo) == [1, 0] and n[0] == 1


def test_exact_sum_is_the_rounded_fixed_point_sum():
    # the definition written out with rationals: sum of floor(t 2^100),
    # divided by 2^100 and rounded once (Fraction -> float rounds to nearest)
    from fractions import Fraction
    rng = np.random.default_rng(11)
    cases = [np.exp(rng.standard_normal(n) * s) for n, s in ((1, 1), (7, 3), (64, 0.5), (300, 8))]
    cases = [c / c.max() for c in cases]
    cases += [np.array([1.0, 2.0 ** -100, 2.0 ** -101, 5e-324, 0.0]),
              np.array([1.0, 2.0 ** -53, 2.0 ** -53]),
              np.array([1.0, 2.0 ** -53, 2.0 ** -100])]
    for t in cases:
        want = float(Fraction(sum(math.floor(Fraction(v) * 2 ** 100) for v in t.tolist()), 2 ** 100))
        assert U.exact_sum(t) == want
        # within vocab * 2^-100 of the exactly rounded real sum: one ulp at most
        assert abs(U.exact_sum(t) - math.fsum(t)) <= math.ulp(math.fsum(t))


def test_exact_sum_rounds_ties_to_even():
    # 1 + 2^-53 is halfway between 1 and the next double: ties to even gives 1;
    # any further bit below breaks the tie upwards
    assert U.exact_sum(np.array([1.0, 2.0 ** -53])) == 1.0
    assert U.exact_sum(np.array([1.0, 2.0 ** -53, 2.0 ** -99])) == 1.0 + 2.0 ** -52
    assert U.exact_sum(np.array([1.0, 2.0 ** -52, 2.0 ** -53])) == 1.0 + 2.0 ** -51


def _permuted_rows(seed, vocab):
    """8 rows over `vocab`: rows 1, 3, 4 and 6 are permutations of one
    Gaussian row (tied confidences), rows 0 and 5 are more confident, rows 2
    and 7 less."""
    rng = np.random.default_rng(seed)
    base = (rng.standard_normal(vocab) * 2.0).astype(np.float32)
    rows = np.empty((8, vocab), np.float32)
    for i in (1, 3, 4, 6):
        rows[i] = base[rng.permutation(vocab)]
    for i, peak in ((0, 9.0), (5, 8.0)):
        rows[i] = rng.standard_normal(vocab).astype(np.float32) * 2.0
        rows[i][rng.integers(vocab)] += np.float32(peak)
    for i in (2, 7):
        rows[i] = (rng.standard_normal(vocab) * 0.5).astype(np.float32)
    return rows


def test_permuted_rows_tie_exactly_and_split_by_row_index():
    V = 4096
    x = _permuted_rows(5, V)
    conf = [U.row_confidence(r)[3] for r in x]
    assert conf[1] == conf[3] == conf[4] == conf[6]
    assert min(conf[0], conf[5]) > conf[1] > max(conf[2], conf[7])
    # a plain float64 sum would not tie these rows: its value depends on the order
    plain = {float(np.exp(r.astype(np.float64) - float(r.max())).sum()) for r in x[[1, 3, 4, 6]]}
    assert len(plain) > 1
    # fully-active block: k = ceil(8 / n) rows by (confidence, row index)
    for n, want in ((3, {0, 5, 1}), (2, {0, 5, 1, 3}), (4, {0, 5}), (1, set(range(8)))):
        m, tok, nc, _ = U.unmask_select(x, [0, 8], [U.MODE_FULL], [n], np.float32(0.999),
                                        np.ones(8, np.uint8), np.full(8, -1, np.int32))
        assert set(np.flatnonzero(m == 0)) == want, n
        assert nc[0] == len(want)
    # with rows 0 and 1 already committed the cut falls between rows 3 and 4
    mk = np.ones(8, np.uint8)
    mk[[0, 1]] = 0
    m, _, nc, _ = U.unmask_select(x, [0, 8], [U.MODE_FULL], [2], np.float32(0.999), mk, np.full(8, -1, np.int32))
    assert set(np.flatnonzero(m == 0)) == {0, 1, 5, 3, 4} and nc[0] == 3
