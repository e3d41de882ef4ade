"""Scaffold speculative verification -- oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What is computed (restated from the Fast-dDrive method summary, sec. 3.2,
"Scaffold Speculative Decoding"):
  * scaffold positions of a block are accepted without any check;
  * the MDM head drafts every editable position of the block in one pass;
  * the AR head scores the whole block in one causal pass, giving
    p_AR(. | x_<i) for every position i; walking left to right, a draft token
    equal to the AR argmax is accepted; at the first mismatch the AR's own
    prediction is taken instead (the bonus token, so every round makes
    progress) and the later drafts are dropped.
  * The output is identical to pure greedy AR decoding (Fast-dDrive sec. 1,
    contributions).

Readings: the caller passes logit row i already aligned with draft position i
(row i = p_AR(. | x_<i)); argmax ties resolve to the lowest index; verification
starts at the first unverified row ``first``; when every draft from ``first``
to m - 1 passes, the bonus is the argmax of row m if the logits have that row,
else there is none (-1).
"""

import numpy as np


def argmax_lowest(row):
    """Argmax of a float32 row; ties resolve to the lowest index."""
    row = np.asarray(row, dtype=np.float32)
    return int(np.flatnonzero(row == row.max())[0])


def spec_verify_one(logits, draft, fixed, first):
    """One sequence.  logits [n_lrows][V], draft [m], fixed [m] or None.

    Returns (accept_len, bonus)."""
    n_lrows = logits.shape[0]
    m = len(draft)
    k = first
    while k < m:
        if fixed is not None and fixed[k]:
            k += 1
            continue
        if argmax_lowest(logits[k]) == int(draft[k]):
            k += 1
            continue
        break
    bonus = argmax_lowest(logits[k]) if k < n_lrows else -1
    return k - first, bonus


def spec_verify(logits, draft, fixed, first):
    """Batched: logits [S][n_lrows][V], draft [S][m], fixed [S][m] or None,
    first [S].  Returns (accept_len [S], bonus [S]) as int32 arrays."""
    S = logits.shape[0]
    acc = np.zeros(S, dtype=np.int32)
    bon = np.zeros(S, dtype=np.int32)
    for s in range(S):
        acc[s], bon[s] = spec_verify_one(
            logits[s], draft[s], None if fixed is None else fixed[s], int(first[s]))
    return acc, bon


# ---------------------------------------------------------------------------
# Trajectory-only sampling (Fast-dDrive method summary sec. 3.3, design
# principle one): in the trajectory section the AR verifier samples from
# softmax(l / T) instead of taking its argmax.  The sample is taken with the
# Gumbel-max construction on caller-supplied noise g ~ Gumbel(0, 1):
# argmax_v (l_v / T + g_v) is distributed as softmax(l / T).  Reading: the
# library's definition of the perturbed value is one float32 multiply by
# 1 / T and one float32 add, each rounded to nearest (numpy float32 scalar
# arithmetic is IEEE single precision, so this is that definition).

def perturbed_row(row, noise, inv_temperature):
    """float32 l * inv_temperature + g, each operation rounded to float32."""
    x = np.asarray(row, dtype=np.float32) * np.float32(inv_temperature)
    return (x.astype(np.float32) + np.asarray(noise, dtype=np.float32)).astype(np.float32)


def spec_verify_sampled(logits, noise, inv_temperature, draft, fixed, first):
    """spec_verify with every row's token taken from the perturbed row."""
    pert = np.stack([np.stack([perturbed_row(logits[s, i], noise[s, i], inv_temperature)
                               for i in range(logits.shape[1])]) for s in range(logits.shape[0])])
    return spec_verify(pert, draft, fixed, first)
