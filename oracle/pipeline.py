"""Pipelined parallel decoding schedule -- oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What is scheduled (restated from the Fast-dVLA notes, key design 4, and its
"complete example"):
  * the completion ratio of a block is the fraction of its tokens already
    revealed;
  * when a block's predecessor passes the add threshold, the block joins the
    forward passes as semi-active: it commits only predictions whose
    confidence exceeds the threshold;
  * when the predecessor passes the activation threshold, the block becomes
    fully active: besides the threshold it ranks its remaining positions by
    confidence and commits at least a 1/n fraction of them per step;
  * blocks stay causal across (a later block never changes an earlier one);
    a completed prefix becomes cached and later steps only compute the
    active blocks.

Readings where the notes are silent or their figure is garbled:
  * the first block has no predecessor and is fully active from the start;
    a committed predecessor counts as complete (ratio 1);
  * the notes use one word, "exceeds", for the add threshold, the
    activation threshold and the confidence threshold, so all three compare
    strictly (``exceeds``); the ratio is revealed / size in double
    precision; the add and activation thresholds, the confidence threshold
    and n are parameters (the notes give 0.5 as one model's semi-active
    confidence threshold and no value for the others).  With add = act = 1 a
    block never joins before its predecessor is committed (no overlap);
  * at most `window` blocks are active at once; blocks join in order;
  * transitions are evaluated before each step from the ratios the previous
    steps left; a block that has revealed every token stays in the active set
    (its keys are still needed by later blocks) until every earlier block is
    committed, and blocks are committed strictly in order, right after the
    step that completes them.

``logits_for(b, s)`` supplies block b's float32 logits [rows][V] for its
s-th step as an active block (s = 0, 1, ...), so both sides of a parity test
read the same synthetic model outputs.
"""

import numpy as np

from . import unmask as OU

WAIT, SEMI, FULL = "wait", "semi", "full"


def exceeds(ratio, threshold):
    """A completion ratio passes a threshold only when it is strictly
    above it (the notes' "exceeds")."""
    return ratio > threshold


def pipelined_decode(block_sizes, logits_for, add, act, tau, n_div, window):
    """Run the schedule to completion.

    Returns (tokens, trace): tokens is a list of int32 arrays, one per block;
    trace is one dict per step with the active blocks, their modes, the
    number of rows each committed that step and the blocks committed after
    it."""
    nb = len(block_sizes)
    masked = [np.ones(n, np.uint8) for n in block_sizes]
    tokens = [np.full(n, -1, np.int32) for n in block_sizes]
    state = [WAIT] * nb
    local_step = [0] * nb
    committed = 0            # blocks 0 .. committed - 1 are in the cache
    trace = []

    def ratio(b):
        if b < committed:
            return 1.0
        # revealed / size rounded once: a ratio equal to a threshold stays
        # equal, so it does not exceed it
        return (block_sizes[b] - int(masked[b].sum())) / block_sizes[b]

    while committed < nb:
        # ---- transitions, in block order
        for b in range(committed, nb):
            if b == committed:
                state[b] = FULL          # no pending predecessor
                continue
            if state[b - 1] == WAIT:
                break                    # blocks join in order
            r = ratio(b - 1)
            if state[b] == WAIT:
                n_active = sum(1 for x in range(committed, nb) if state[x] != WAIT)
                if exceeds(r, add) and n_active < window:
                    state[b] = SEMI
            if state[b] == SEMI and exceeds(r, act):
                state[b] = FULL
        active = [b for b in range(committed, nb) if state[b] != WAIT]

        # ---- one denoise step over the active blocks
        lg = np.concatenate([logits_for(b, local_step[b]) for b in active])
        off = np.concatenate([[0], np.cumsum([block_sizes[b] for b in active])]).astype(np.int64)
        modes = [OU.MODE_FULL if state[b] == FULL else OU.MODE_SEMI for b in active]
        divs = [n_div if state[b] == FULL else 1 for b in active]
        m_in = np.concatenate([masked[b] for b in active])
        t_in = np.concatenate([tokens[b] for b in active])
        m_out, t_out, n_commit, _ = OU.unmask_select(lg, off, modes, divs, np.float32(tau), m_in, t_in)
        for j, b in enumerate(active):
            masked[b] = m_out[off[j]:off[j + 1]].copy()
            tokens[b] = t_out[off[j]:off[j + 1]].copy()
            local_step[b] += 1

        # ---- in-order commit of completed blocks
        done = []
        while committed < nb and state[committed] != WAIT and masked[committed].sum() == 0:
            done.append(committed)
            committed += 1
        trace.append(dict(active=list(active), modes=[state[b] for b in active],
                          n_commit=[int(x) for x in n_commit], committed=done))
    return tokens, trace
