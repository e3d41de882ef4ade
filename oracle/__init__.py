"""CPU oracle for the block-causal masked-diffusion denoising step.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously-correct
NumPy float64 restatement of what the GPU library computes.  Only the test
suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import it.  It shares no code with the HIP library or its Python binding
and imports nothing from them; inputs reach it as plain NumPy arrays.

Modules
  attention  explicit-mask block-causal GQA attention (cached prefix, active
             blocks, optional shared-prefix fork) and a full-sequence
             formulation used to pin it
  kvcache    in-order append of completed blocks to a per-sequence cache
  unmask     per-row max / argmax / softmax confidence and the threshold +
             ceil(remaining / n) fallback selection
  verify     left-to-right speculative verification (accept length + bonus),
             and its sampled form (Gumbel-max over supplied noise)
  pipeline   the pipelined parallel decoding schedule (semi / fully active
             blocks, add and activation thresholds, in-order commit)
  section    the Section Diffusion decode schedule (block or section
             visibility units, scaffold rows never masked, fixed steps)
  trajectory the shared-prefix fork decoding a whole trajectory section with
             scaffold speculative rounds (draft, verify, bonus, finished
             rollouts leaving, private commits)

Sources (the pages the method is described on):
  * "Fast-dDrive" (Chinese translation of arXiv 2605.23163): abstract, sec. 1
    and sec. 2 (block diffusion, scaffold speculative decoding, shared-prefix
    fork).
  * WAM-Diff2 press article, sec. 2.1 "Block-Causal attention" (B = 1 equals
    autoregressive decoding) and sec. 3 (system acceleration).
  * Fast-dVLA reading notes, "Key designs" 1 (block-causal attention) and 4
    (pipelined parallel decoding, semi/fully-active commit rule).
  * Fast-dDrive method summary, sec. 3.1 (block-causal MDM), sec. 3.2
    (scaffold, section table, Section Diffusion and Scaffold Speculative
    decoding) and sec. 3.3 (shared-prefix rollouts).

Parity status: every function here is pinned by tests in ``tests/`` against
closed forms, invariants the pages state, brute force on tiny inputs or an
independent library routine; none is "parity unpinned".
"""

from . import attention, kvcache, unmask, verify  # noqa: F401

__all__ = ["attention", "kvcache", "unmask", "verify"]
