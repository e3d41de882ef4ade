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
    i.e. 1 / sum_j exp(l_j - max_j l_j);
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

import numpy as np

MODE_SEMI = 0
MODE_FULL = 1


def row_confidence(row):
    """(max, argmax, sum_exp, confidence) of one float32 logit row."""
    row = np.asarray(row, dtype=np.float32)
    m = row.max()
    a = int(np.flatnonzero(row == m)[0])
    s = float(np.exp(row.astype(np.float64) - np.float64(m)).sum())
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
