"""Confidence-threshold unmask with the ceil(remaining / n) fallback -- oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What is computed (restated from the pages):
  * A masked-diffusion step predicts every still-masked position and reveals
    some of them; a revealed token never changes again (Fast-dDrive method
    summary sec. 3.1; Fast-dVLA notes, key design 2).
  * Fast-dVLA notes, key design 4 (pipelined parallel decoding): a
    semi-active block commits only the positions whose prediction
    confidence exceeds the threshold; a fully-active block also ranks the
    remaining positions by confidence and commits at least a 1/n fraction of
    them every step.

Readings where the pages are silent or vague:
  * confidence = the largest softmax probability of the row at temperature 1,
    i.e. 1 / sum_j exp(l_j - max_j l_j).  The sum is taken exactly, so that it
    does not depend on the order of the terms: each float64 term
    exp(l_j - max) (in [0, 1]) is cut to a multiple of 2^-100, the multiples
    are added as integers, and the total is rounded once to float64.  (Two
    rows whose logits are permutations of each other then have equal
    confidences, and their order is the row index, whatever order a sum runs
    in.  The cut changes each term by less than 2^-100, the sum by less than
    vocab * 2^-100.)
  * "exceeds" is a strict comparison, conf > tau, with tau the float32
    threshold promoted exactly to float64;
  * FULL commits k = min(|E|, max(|A|, ceil(|E| / n))) rows of the block's
    masked set E, where A = {r in E : conf_r > tau}; SEMI commits k = |A|;
    the k rows are the first k of E ordered by (confidence descending, row
    index ascending);
  * argmax ties resolve to the lowest vocabulary index;
  * n is supplied per block (the number of denoise steps left in the block's
    fixed step budget, so a block always completes within its budget).

Precision: the maximum and argmax are exact comparisons of the float32
logits; the sum of exponentials and the confidence are float64.  All
selection decisions are taken on these float64 confidences.
"""

import math

import numpy as np

MODE_SEMI = 0
MODE_FULL = 1


FIXED_BITS = 100   # the sum's terms are cut to multiples of 2^-FIXED_BITS


def exact_sum(terms):
    """sum(terms) for float64 terms in [0, 1], order-independent: the exact
    integer sum of floor(t * 2^FIXED_BITS), rounded once to float64, times
    2^-FIXED_BITS."""
    t = np.asarray(terms, dtype=np.float64)
    f, ex = np.frexp(t)                                  # t = f 2^ex, f in [0.5, 1) (0 for t = 0)
    mant = (f * 2.0 ** 53).astype(np.uint64)             # t = mant 2^(ex - 53), mant < 2^53
    shift = ex.astype(np.int64) + (FIXED_BITS - 53)      # floor(t 2^FIXED_BITS) = floor(mant 2^shift)
    total = 0
    for k in range(4):                                   # 32-bit limbs of the fixed-point value
        r = 32 * k - shift                               # the limb holds bits r .. r + 31 of mant
        down = np.right_shift(mant, np.clip(r, 0, 63).astype(np.uint64))
        up = np.left_shift(mant, np.clip(-r, 0, 63).astype(np.uint64))
        limb = np.where(r >= 0, down, up) & np.uint64(0xFFFFFFFF)
        limb = np.where(r >= 64, np.uint64(0), limb)
        total += int(limb.sum(dtype=np.uint64)) << (32 * k)
    return math.ldexp(float(total), -FIXED_BITS)         # int -> float rounds to nearest even


def row_confidence(row):
    """(max, argmax, sum_exp, confidence) of one float32 logit row."""
    row = np.asarray(row, dtype=np.float32)
    m = row.max()
    a = int(np.flatnonzero(row == m)[0])
    s = exact_sum(np.exp(row.astype(np.float64) - np.float64(m)))
    return float(m), a, s, 1.0 / s


def commit_count(n_masked, n_above, mode, n_div):
    """How many masked rows of a block are committed this step."""
    if mode == MODE_SEMI:
        return n_above
    if mode == MODE_FULL:
        fallback = -(-n_masked // n_div)          # ceil(|E| / n)
        return min(n_masked, max(n_above, fallback))
    raise ValueError("unknown unmask mode %r" % (mode,))


def unmask_select(logits, blk_off, mode, n_div, threshold, masked, tokens):
    """One unmask step over the active rows.

    logits [R][V] float32; blk_off [n_blk + 1]; mode, n_div [n_blk];
    threshold a float32 value; masked [R] (1 = still masked), tokens [R].

    Returns (masked_out, tokens_out, n_commit [n_blk], conf [R] float64 with
    NaN on rows that were not masked on entry).
    """
    logits = np.asarray(logits, dtype=np.float32)
    masked_out = np.array(masked, dtype=np.uint8)
    tokens_out = np.array(tokens, dtype=np.int32)
    R = logits.shape[0]
    tau = float(np.float32(threshold))
    conf = np.full(R, np.nan)
    argmax = np.full(R, -1, dtype=np.int64)
    for r in range(R):
        if masked_out[r]:
            _, argmax[r], _, conf[r] = row_confidence(logits[r])
    n_blk = len(blk_off) - 1
    n_commit = np.zeros(n_blk, dtype=np.int32)
    for b in range(n_blk):
        rows = [r for r in range(blk_off[b], blk_off[b + 1]) if masked_out[r]]
        n_above = sum(1 for r in rows if conf[r] > tau)
        k = commit_count(len(rows), n_above, mode[b], int(n_div[b]))
        ranked = sorted(rows, key=lambda r: (-conf[r], r))
        for r in ranked[:k]:
            tokens_out[r] = argmax[r]
            masked_out[r] = 0
        n_commit[b] = k
    return masked_out, tokens_out, n_commit, conf
