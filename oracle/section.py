"""Section Diffusion decode schedule -- oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What is computed (restated from the Fast-dDrive method summary, sec. 3.1 on
semantically aligned blocks and sec. 3.2 "Section Diffusion"):
  * the output is a sequence of sections decoded in causal order; each
    section's editable tokens are cut into ceil(|E_s| / d) blocks;
  * the prefilled scaffold (template) tokens sit among the editable ones and
    are never masked, never predicted and never changed;
  * a block is denoised for a fixed number of steps; each step is one
    attention pass of the active rows over the cached prefix, then a
    confidence unmask over the block's still-masked editable rows
    (threshold, plus at least ceil(remaining / steps left));
  * completed context is reused from the KV cache instead of being
    recomputed.

The visibility unit is a parameter:
  * block units (WAM-Diff2 sec. 2.1; Fast-dVLA key design 1): a block sees
    the prefix, every earlier block and itself; its K/V are committed when it
    completes;
  * section units (method summary sec. 3.1): the blocks of one section see
    each other bidirectionally and later sections see only completed earlier
    sections.  Every row of the section is therefore active in each step of
    each of its blocks (their keys are in the current block's view and change
    with the section), and the section's K/V are committed when its last
    block completes.

Readings: the K/V committed for a unit are those of its last step (the
pages do not say which forward produces them); n = steps left in the block's
fixed budget, so a block's editable rows are all revealed within it.
"""

import numpy as np

from . import attention as OA, kvcache as OK, unmask as OU


def section_decode(prefix_k, prefix_v, prefix_len, units, blocks, inputs, steps, tau, masked0, tokens0,
                   scale=None, keep=(), attend_all=True, trace=None):
    """Decode one sequence.

    prefix_k/v [Hkv][>= prefix_len][D]; ``units`` lists the block indices of
    each visibility unit in order (consecutive blocks); ``blocks`` holds the
    rows of every block; ``inputs(b, st)`` returns block b's step-st model
    outputs as float32 arrays (q [1][unit rows][Hq][D], k / v
    [1][Hkv][unit rows][D] for all rows of b's unit, logits [rows of b][V]);
    masked0 / tokens0 [all output rows] give the initial state (scaffold rows
    unmasked, with their tokens).

    Returns dict(tokens, masked, n_commit [block][step], cache_k, cache_v,
    attention {(b, st): float64 [1][unit rows][Hq][D] for (b, st) in keep}).
    The synthetic logits do not depend on the attention outputs, so with
    attend_all False only the kept steps' attention is computed (same
    results, less work).  With ``trace`` a list, every unmask step appends
    (block, step, float64 confidences of the block's rows with NaN on rows
    revealed before the step, commit count).
    """
    cache = OK.new_cache(np.asarray(prefix_k)[None], np.asarray(prefix_v)[None], [prefix_len])
    masked = np.array(masked0, np.uint8)
    tokens = np.array(tokens0, np.int32)
    row0 = np.concatenate([[0], np.cumsum(blocks)]).astype(np.int64)
    n_commit = [[] for _ in blocks]
    kept = {}
    for unit in units:
        unit_rows = sum(blocks[b] for b in unit)
        for b in unit:
            r0, r1 = row0[b], row0[b + 1]
            for st in range(steps):
                q, k, v, lg = inputs(b, st)
                if q.shape[1] != unit_rows:
                    raise ValueError("block %d: inputs hold %d rows, its unit %d" % (b, q.shape[1], unit_rows))
                if attend_all or (b, st) in keep:
                    ck, cv = cache[0]
                    o = OA.attention_step(q, ck[None], cv[None], [ck.shape[1]], k, v, [0, unit_rows],
                                          OA.MASK_BIDIR, scale=scale)
                    if (b, st) in keep:
                        kept[(b, st)] = o
                m, t, n, conf = OU.unmask_select(lg, [0, r1 - r0], [OU.MODE_FULL], [steps - st], np.float32(tau),
                                                 masked[r0:r1], tokens[r0:r1])
                if trace is not None:
                    trace.append((b, st, conf, int(n[0])))
                masked[r0:r1], tokens[r0:r1] = m, t
                n_commit[b].append(int(n[0]))
        OK.commit(cache, 0, cache[0][0].shape[1], k[0], v[0])
    return dict(tokens=tokens, masked=masked, n_commit=n_commit, cache_k=cache[0][0], cache_v=cache[0][1],
                attention=kept)
