"""Host decode schedules driving the C-ABI calls.

Every step of the path runs in the HIP kernels behind ``binding``; this
module only owns device buffers and issues the calls in the order the pages
describe:

* ``SectionDecode`` -- Section Diffusion (Fast-dDrive method summary,
  sec. 3.1 - 3.2): output blocks are decoded in causal order over a
  committed prefix; each block takes a fixed number of denoise steps
  (attention, then confidence unmask with n = steps left), and its K/V are
  committed to the cache when it completes -- or, with section visibility,
  when its section does.  Optionally the sections' scaffold rows sit inside
  the blocks.  Also the large-block decode at batch > 1 (one
  attention call covers every sequence; the unmask call sees one block per
  sequence).
* ``ForkVerify`` -- shared-prefix fork with scaffold speculative decoding
  (method summary sec. 3.2 - 3.3): N rollouts share one prefix cache; per
  trajectory block and round, a bidirectional draft pass, a draft argmax
  (threshold 0 reveals every masked row), a causal verify pass and the
  verify call.
* ``PipelinedDecode`` -- pipelined parallel decoding (Fast-dVLA notes, key
  design 4): up to ``window`` consecutive blocks denoised together, later
  ones semi-active until their predecessor is far enough along; one
  attention call and one unmask call per step, in-order commits.

The model between attention and logits is not part of this library:
attention outputs are produced and discarded, logits and the active rows'
Q/K/V are seeded synthetic tensors made up-front and resident on the GPU.
"""

import numpy as np
import torch

from . import binding as B
from . import synth


class SectionDecode:
    """Section Diffusion (Fast-dDrive method summary sec. 3.1 - 3.2): blocks
    decoded in causal order over a committed prefix, a fixed number of
    denoise steps each (attention, then confidence unmask with n = steps
    left).

    ``visibility`` picks the unit that is bidirectional and committed whole:
      * "block": a block sees the prefix, earlier blocks and itself, and is
        committed when it completes;
      * "section": the blocks of one section see each other, so every row of
        the section is active in each step of each of its blocks (attention
        over the section's rows, unmask over the current block's rows) and
        the section is committed when its last block completes.
    With a preset that sets ``scaffold``, the blocks hold the sections'
    scaffold rows among the editable ones (``synth.section_layout``); they
    start unmasked with their template tokens, so the unmask never counts,
    ranks or changes them.

    Also the large-block decode at batch > 1 (one attention call covers
    every sequence; the unmask call sees one block per sequence).

    ``mask`` is the in-block mode of the attention calls (bidirectional by
    default; causal gives the AR form of the same schedule).  With
    ``logits_pool`` / ``qkv_pool`` = k, k distinct seeded logits / Q-K-V sets
    are drawn and cycled over the (block, step) pairs instead of one per
    pair, which bounds the host time and memory of long, wide decodes."""

    def __init__(self, preset, seed=0, n_seq=None, device="cuda:0", logits_pool=None,
                 planted_frac=0.0, planted_delta=12.0, visibility="block", mask=None, qkv_pool=None):
        p = dict(preset)
        self.p = p
        self.S = n_seq or p.get("n_seq", 1)
        self.Hq, self.Hkv, self.D = p["n_q_heads"], p["n_kv_heads"], p["head_dim"]
        self.dtype = p["dtype"]
        self.steps = p["steps"]
        self.V, self.sigma, self.tau = p["vocab"], p["sigma"], p["threshold"]
        self.prefix = p["prefix"]
        self.dev = device
        editable = None
        if p.get("scaffold"):
            lay = synth.section_layout(p.get("layout_seed", 0))
            self.blocks = [b for sec in lay for b in sec["blocks"]]
            per_section = [len(sec["blocks"]) for sec in lay]
            editable = np.concatenate([sec["kinds"] for sec in lay])
        else:
            self.blocks = list(p["blocks"])
            per_section = list(p.get("sections", [len(self.blocks)]))
        nb = len(self.blocks)
        if visibility == "block":
            self.units = [[b] for b in range(nb)]
        elif visibility == "section":
            if sum(per_section) != nb:
                raise ValueError("the preset's sections do not cover its blocks")
            first = np.concatenate([[0], np.cumsum(per_section)])
            self.units = [list(range(first[i], first[i + 1])) for i in range(len(per_section))]
        else:
            raise ValueError("visibility must be 'block' or 'section'")
        self.visibility = visibility
        self.unit_of = {b: u for u, blks in enumerate(self.units) for b in blks}
        self.unit_rows = [sum(self.blocks[b] for b in blks) for blks in self.units]
        self.row0 = [0] + [int(x) for x in np.cumsum(self.blocks)]
        self.cap = self.prefix + sum(self.blocks)
        S, Hkv, D = self.S, self.Hkv, self.D
        tdt = synth.torch_dtype(self.dtype)
        (k, v), _ = synth.kv_cache(seed, S, Hkv, self.cap, D, [self.prefix] * S, self.dtype)
        self.cache = B.KVCache(k.to(device), v.to(device))
        self.len0 = np.full(S, self.prefix, np.int32)
        # per (block, step) the active rows (those of the block's unit) and
        # the block's logits, resident on the device; with logits_pool = k,
        # k distinct logits tensors are cycled instead
        bmax = max(self.blocks)
        self.mask = B.BC_MASK_BLOCK_BIDIR if mask is None else mask
        self.qkv_pool = qkv_pool
        drawn = {}
        self.qkv = []
        for b, bs in enumerate(self.blocks):
            ur = self.unit_rows[self.unit_of[b]]
            row = []
            for st in range(self.steps):
                key = self.qkv_index(b, st)
                if key not in drawn:
                    (qt, _), (kt, _), (vt, _) = synth.active_qkv(seed, S, ur, self.Hq, Hkv, D, self.dtype, *key)
                    drawn[key] = (qt.to(device), kt.to(device), vt.to(device))
                row.append(drawn[key])
            self.qkv.append(row)

        def make_logits(rows, *idx):
            x = synth.logits(seed, rows, self.V, self.sigma, *idx)
            if planted_frac:
                synth.plant_peaks(x, seed, planted_frac, planted_delta, *idx)
            return torch.from_numpy(x).to(device)

        if logits_pool:
            pool = [make_logits(S * bmax, 1000 + i) for i in range(logits_pool)]
            self.logits = [[pool[(b * self.steps + st) % logits_pool][: S * bs] for st in range(self.steps)]
                           for b, bs in enumerate(self.blocks)]
        else:
            self.logits = [[make_logits(S * bs, b, st) for st in range(self.steps)]
                           for b, bs in enumerate(self.blocks)]
        self.out = {ur: torch.empty((S, ur, self.Hq, D), dtype=tdt, device=device) for ur in set(self.unit_rows)}
        n_rows = S * sum(self.blocks)
        self.masked = torch.ones(n_rows, dtype=torch.uint8, device=device)
        self.tokens = torch.full((n_rows,), -1, dtype=torch.int32, device=device)
        # initial state of every block's rows, laid out [block][seq][row]
        self.masked0 = self.tokens0 = None
        if editable is not None:
            tmpl = synth.scaffold_tokens(p.get("layout_seed", 0), len(editable), self.V)
            m0 = np.concatenate([np.tile(editable[self.row0[b]:self.row0[b + 1]], S) for b in range(nb)])
            t0 = np.concatenate([np.tile(np.where(editable == 0, tmpl, -1)[self.row0[b]:self.row0[b + 1]], S)
                                 for b in range(nb)]).astype(np.int32)
            self.masked0 = torch.from_numpy(m0).to(device)
            self.tokens0 = torch.from_numpy(t0).to(device)
        self.conf = torch.empty(S * bmax, dtype=torch.float32, device=device)
        self.n_commit = torch.zeros(self.S, dtype=torch.int32, device=device)
        self.ws_attn = torch.zeros(max(B.bc_attn_workspace_bytes(self.cache, None, (S, ur, self.Hq, D), [0, ur])
                                       for ur in set(self.unit_rows)), dtype=torch.uint8, device=device)
        self.ws_unmask = torch.zeros(B.bc_unmask_workspace_bytes(S * bmax, self.V), dtype=torch.uint8,
                                     device=device)
        self.scale = 1.0 / np.sqrt(D)
        self.hooks = None   # optional callables around each call: hooks(kind, "pre"/"post")
        self.after_attn = None   # optional after_attn(b, st, out), called after each attention call

    def qkv_index(self, b, st):
        """Seed indices of block b's step-st Q/K/V draw."""
        if not self.qkv_pool:
            return (b, st)
        return (2000 + self.unit_rows[self.unit_of[b]], (b * self.steps + st) % self.qkv_pool)

    @property
    def tokens_per_decode(self):
        """Decoded (editable) tokens per decode, all sequences."""
        if self.masked0 is None:
            return self.S * sum(self.blocks)
        return int(self.masked0.sum())

    @property
    def denoise_steps(self):
        return len(self.blocks) * self.steps

    def _hook(self, kind, when):
        if self.hooks is not None:
            self.hooks(kind, when)

    def run(self, stream=None):
        """One whole decode.  Returns nothing; tokens / masked hold the result."""
        S = self.S
        length = self.len0.copy()
        # every output row starts masked (scaffold rows revealed with their
        # template tokens): one launch for the whole decode, before its first
        # block; a block's rows are not touched before the block runs
        if self.masked0 is None:
            self.masked.fill_(1)
        else:
            self.masked.copy_(self.masked0)
            self.tokens.copy_(self.tokens0)
        for u, blks in enumerate(self.units):
            ur = self.unit_rows[u]
            out = self.out[ur]
            for b in blks:
                bs, off = self.blocks[b], self.row0[b]
                rows = slice(S * off, S * (off + bs))
                masked, tokens = self.masked[rows], self.tokens[rows]
                blk_rows = list(range(0, S * bs + 1, bs))
                for st in range(self.steps):
                    q, k, v = self.qkv[b][st]
                    self._hook("attn", "pre")
                    B.bc_attn_step(self.cache, length, None, None, q, k, v, [0, ur], self.mask,
                                   self.scale, out, self.ws_attn, stream=stream)
                    self._hook("attn", "post")
                    if self.after_attn is not None:
                        self.after_attn(b, st, out)
                    self._hook("unmask", "pre")
                    B.bc_unmask_select(self.logits[b][st], blk_rows, [B.BC_UNMASK_FULL] * S,
                                       [self.steps - st] * S, self.tau, masked, tokens, self.conf[: S * bs],
                                       self.n_commit[:S], self.ws_unmask, stream=stream)
                    self._hook("unmask", "post")
            q, k, v = self.qkv[blks[-1]][self.steps - 1]
            self._hook("commit", "pre")
            # every sequence has the same length: one commit of all of them
            B.bc_kv_commit(self.cache, length, B.BC_ALL_SEQ, int(length[0]), ur, k, v, stream=stream)
            self._hook("commit", "post")


class ForkVerify:
    """One round of the shared-prefix fork with scaffold speculative
    decoding for one trajectory block (Fast-dDrive method summary sec. 3.2,
    3.3): N rollouts share one prefix cache and keep their earlier trajectory
    blocks in private caches.  A round is

      1. draft pass: bidirectional attention of the block's rows;
      2. draft argmax: an unmask with threshold 0 and SEMI mode reveals every
         masked row, token = argmax of its draft logits; the block's scaffold
         rows (one template for all rollouts) start unmasked with their
         template tokens, so only the editable rows are drafted;
      3. verify pass: causal attention of the same rows;
      4. speculative verify of the drafts against the verify logits, scaffold
         rows accepted as they are; with a temperature, the verify samples
         its tokens (trajectory-only sampling, sec. 3.3) by Gumbel-max over
         seeded per-rollout noise.

    Logits, the rows' Q/K/V and the private caches are seeded synthetic
    tensors made up-front and resident on the device; the drafts the verify
    call checks are the tokens step 2 produced."""

    def __init__(self, n_rollouts, seed=0, device="cuda:0", block=0, scaffold_frac=0.3, preset=None,
                 temperature=None):
        p = dict(preset or synth.PRESETS["fork"])
        self.N = n_rollouts
        self.Hq, self.Hkv, self.D = p["n_q_heads"], p["n_kv_heads"], p["head_dim"]
        self.dtype = p["dtype"]
        self.prefix = p["prefix"]
        self.V, self.sigma = p["vocab"], p["sigma"]
        blocks = list(p["blocks"])
        self.R = blocks[block]
        self.priv_len = [sum(blocks[:block])] * n_rollouts
        self.priv_cap = max(sum(blocks[:-1]), 1)
        self.dev = device
        N, R, Hq, Hkv, D = self.N, self.R, self.Hq, self.Hkv, self.D
        (pk, pv), _ = synth.kv_cache(seed, 1, Hkv, self.prefix, D, [self.prefix], self.dtype)
        self.shared = B.KVCache(pk.to(device), pv.to(device))
        (vk, vv), _ = synth.kv_cache(seed, N, Hkv, self.priv_cap, D, self.priv_len, self.dtype,
                                     purpose=("priv_k", "priv_v"))
        self.priv = B.KVCache(vk.to(device), vv.to(device))
        self.qkv = {}
        for pass_id in (0, 1):   # draft, verify
            (q, _), (k, _), (v, _) = synth.active_qkv(seed, N, R, Hq, Hkv, D, self.dtype, 100 + block, pass_id)
            self.qkv[pass_id] = (q.to(device), k.to(device), v.to(device))
        self.draft_logits = torch.from_numpy(synth.logits(seed, N * R, self.V, self.sigma, 200 + block)).to(device)
        self.verify_logits = torch.from_numpy(
            synth.logits(seed, N * R, self.V, self.sigma, 300 + block)).to(device).view(N, R, self.V)
        # the block's scaffold rows: one prefilled template shared by every
        # rollout, accepted as they are; only the editable rows are drafted
        fixed, tmpl = self._scaffold(seed, block, scaffold_frac)
        self.scaffold_frac = scaffold_frac
        self.fixed = torch.from_numpy(fixed).to(device)
        self.masked0 = torch.from_numpy((1 - fixed).reshape(-1)).to(device)
        self.tokens0 = torch.from_numpy(np.where(fixed == 1, tmpl, -1).astype(np.int32).reshape(-1)).to(device)
        # trajectory-only sampling (method summary sec. 3.3): the verify
        # samples softmax(l / T) through Gumbel-max on per-rollout noise
        self.temperature = temperature
        self.noise = None
        if temperature is not None:
            self.noise = torch.from_numpy(synth.gumbel(seed, (N, R, self.V), 500 + block)).to(device)
        tdt = synth.torch_dtype(self.dtype)
        self.out = torch.empty((N, R, Hq, D), dtype=tdt, device=device)
        self.masked = torch.ones(N * R, dtype=torch.uint8, device=device)
        self.tokens = torch.full((N * R,), -1, dtype=torch.int32, device=device)
        self.n_commit = torch.zeros(N, dtype=torch.int32, device=device)
        self.first = torch.zeros(N, dtype=torch.int32, device=device)
        self.accept_len = torch.zeros(N, dtype=torch.int32, device=device)
        self.bonus = torch.zeros(N, dtype=torch.int32, device=device)
        self.ws_attn = torch.zeros(B.bc_attn_workspace_bytes(self.shared, self.priv, (N, R, Hq, D), [0, R]),
                                   dtype=torch.uint8, device=device)
        self.ws_unmask = torch.zeros(B.bc_unmask_workspace_bytes(N * R, self.V), dtype=torch.uint8, device=device)
        self.ws_verify = torch.zeros(B.bc_verify_workspace_bytes(N, R, self.V), dtype=torch.uint8, device=device)
        self.scale = 1.0 / np.sqrt(D)
        self.blk_rows = list(range(0, N * R + 1, R))

    def _scaffold(self, seed, block, frac):
        """(fixed [N][R] uint8, template tokens [N][R]) of the block."""
        g = synth.rng(seed, "misc", 400 + block)
        fixed = np.tile((g.random(self.R) < frac).astype(np.uint8), (self.N, 1))
        return fixed, np.tile(synth.scaffold_tokens(seed, self.R, self.V, 400 + block), (self.N, 1))

    def host_inputs(self, seed=0, block=0):
        """The float32 host arrays the device tensors were made from (same
        seeded draws), for checks against the CPU oracle."""
        N, R, Hq, Hkv, D = self.N, self.R, self.Hq, self.Hkv, self.D
        _, (pk, pv) = synth.kv_cache(seed, 1, Hkv, self.prefix, D, [self.prefix], self.dtype)
        _, (vk, vv) = synth.kv_cache(seed, N, Hkv, self.priv_cap, D, self.priv_len, self.dtype,
                                     purpose=("priv_k", "priv_v"))
        qkv = {}
        for pass_id in (0, 1):
            (_, q), (_, k), (_, v) = synth.active_qkv(seed, N, R, Hq, Hkv, D, self.dtype, 100 + block, pass_id)
            qkv[pass_id] = (q, k, v)
        noise = None
        if self.temperature is not None:
            noise = synth.gumbel(seed, (N, R, self.V), 500 + block)
        fixed, tmpl = self._scaffold(seed, block, self.scaffold_frac)
        return dict(pk=pk, pv=pv, vk=vk, vv=vv, qkv=qkv, noise=noise,
                    draft_logits=synth.logits(seed, N * R, self.V, self.sigma, 200 + block),
                    verify_logits=synth.logits(seed, N * R, self.V, self.sigma, 300 + block).reshape(N, R, self.V),
                    fixed=fixed, tokens0=np.where(fixed == 1, tmpl, -1).astype(np.int32).reshape(-1))

    def attention(self, pass_id, stream=None):
        q, k, v = self.qkv[pass_id]
        mask = B.BC_MASK_BLOCK_BIDIR if pass_id == 0 else B.BC_MASK_BLOCK_CAUSAL
        B.bc_attn_step(self.shared, [self.prefix], self.priv, self.priv_len, q, k, v, [0, self.R], mask,
                       self.scale, self.out, self.ws_attn, stream=stream)

    def draft_argmax(self, stream=None):
        self.masked.copy_(self.masked0)
        self.tokens.copy_(self.tokens0)
        B.bc_unmask_select(self.draft_logits, self.blk_rows, [B.BC_UNMASK_SEMI] * self.N, [1] * self.N, 0.0,
                           self.masked, self.tokens, None, self.n_commit, self.ws_unmask, stream=stream)

    def verify(self, stream=None):
        if self.noise is not None:
            B.bc_spec_verify_sampled(self.verify_logits, self.noise, 1.0 / self.temperature,
                                     self.tokens.view(self.N, self.R), self.fixed, self.first, self.accept_len,
                                     self.bonus, self.ws_verify, stream=stream)
        else:
            B.bc_spec_verify(self.verify_logits, self.tokens.view(self.N, self.R), self.fixed, self.first,
                             self.accept_len, self.bonus, self.ws_verify, stream=stream)

    def run(self, stream=None):
        self.attention(0, stream)
        self.draft_argmax(stream)
        self.attention(1, stream)
        self.verify(stream)

    def attention_flops(self, pass_id):
        """4 D Hq per visible (query row, key) pair, the causal in-block
        triangle counted as visible pairs only."""
        R, N = self.R, self.N
        vis = 0
        for s in range(N):
            base = self.prefix + self.priv_len[s]
            vis += R * base + (R * R if pass_id == 0 else R * (R + 1) // 2)
        return 4 * self.D * self.Hq * vis


class ForkTrajectory:
    """Shared-prefix fork decoding a whole trajectory section with scaffold
    speculative rounds (Fast-dDrive method summary sec. 3.2 "Scaffold
    Speculative Decoding", sec. 3.3).

    N rollouts share one prefix cache and decode the section's blocks in
    order.  A block is decoded in rounds; a round runs, for the rollouts that
    have not completed the block, in slot order (the active rollouts, lowest
    first):
      1. draft pass: bidirectional attention of the block's rows over the
         shared prefix and each rollout's private cache;
      2. draft argmax: an unmask with threshold 0 (SEMI) reveals every
         unverified row with the argmax of its draft logits;
      3. verify pass: causal attention of the same rows;
      4. speculative verify from each rollout's first unverified row: the
         accept length and the bonus token.
    The host reads the accept lengths, bonuses and drafts back (one
    synchronisation per round), advances each rollout's first unverified row
    and drops the rollouts that completed the block; their private caches are
    compacted into slot order for the next round.  When every rollout has
    completed the block, each commits it to its private cache with
    bc_kv_commit (the K/V of its last verify pass) and the next block starts.

    The synthetic model outputs of a round (block b, round r):
      * Q/K/V of both passes: seeded draws per (b, r mod ``pool``, pass), one
        slice per slot;
      * logits: a seeded clipped-normal base per kind (draft / verify), whose
        first (active rollouts x rows) rows are the round's logits, with a
        planted argmax per row (value 7 sigma + margin): the verify targets
        t = ``synth.round_targets`` per (b, r, rollout) and the drafts
        ``synth.drafts_with_agreement`` of t at rate ``p_agree``.  The planted
        values are written before the round and restored after it."""

    def __init__(self, n_rollouts, p_agree, seed=0, device="cuda:0", preset=None, pool=2):
        p = dict(preset or synth.PRESETS["fork"])
        self.N, self.p_agree, self.seed, self.pool, self.dev = int(n_rollouts), float(p_agree), seed, pool, device
        self.Hq, self.Hkv, self.D = p["n_q_heads"], p["n_kv_heads"], p["head_dim"]
        self.dtype, self.prefix = p["dtype"], p["prefix"]
        self.V, self.sigma = p["vocab"], p["sigma"]
        self.peak = np.float32(7.0 * self.sigma + p.get("margin", 1.0))
        self.blocks = list(p["blocks"])
        N, Hq, Hkv, D, V = self.N, self.Hq, self.Hkv, self.D, self.V
        self.Rmax = Rmax = max(self.blocks)
        self.cap = sum(self.blocks)
        (pk, pv), _ = synth.kv_cache(seed, 1, Hkv, self.prefix, D, [self.prefix], self.dtype)
        self.shared = B.KVCache(pk.to(device), pv.to(device))
        tdt = synth.torch_dtype(self.dtype)
        z = lambda: torch.zeros((N, Hkv, self.cap, D), dtype=tdt, device=device)
        self.priv = B.KVCache(z(), z())
        self.sub = B.KVCache(z(), z())            # active rollouts' private caches, slot order
        self.priv_len = np.zeros(N, np.int32)
        self.qkv = {}
        for b, R in enumerate(self.blocks):
            for k in range(pool):
                for pass_id in (0, 1):
                    (q, _), (kk, _), (v, _) = synth.active_qkv(seed, N, R, Hq, Hkv, D, self.dtype, 100 + b,
                                                               pass_id, k)
                    self.qkv[(b, k, pass_id)] = (q.to(device), kk.to(device), v.to(device))
        n_logits = N * Rmax * V
        self.base = {kind: torch.from_numpy(synth.clipped_logits(seed, n_logits, self.sigma, 600 + i)).to(device)
                     for i, kind in enumerate(("draft", "verify"))}
        self.out = torch.empty(N * Rmax * Hq * D, dtype=tdt, device=device)
        self.masked = torch.zeros(N * Rmax, dtype=torch.uint8, device=device)
        self.tokens = torch.full((N * Rmax,), -1, dtype=torch.int32, device=device)
        self.first = torch.zeros(N, dtype=torch.int32, device=device)
        self.accept_len = torch.zeros(N, dtype=torch.int32, device=device)
        self.bonus = torch.zeros(N, dtype=torch.int32, device=device)
        self.n_commit = torch.zeros(N, dtype=torch.int32, device=device)
        # each rollout's K/V of its last verify pass in the current block,
        # [N][Hkv][R_b][D] at the front of a flat buffer
        self.last_k = torch.zeros(N * Hkv * Rmax * D, dtype=tdt, device=device)
        self.last_v = torch.zeros_like(self.last_k)
        ws = 0
        for R in set(self.blocks):
            for n in range(1, N + 1):
                ws = max(ws, B.bc_attn_workspace_bytes(self.shared, B.KVCache(self.sub.k[:n], self.sub.v[:n]),
                                                       (n, R, Hq, D), [0, R]))
        self.ws_attn = torch.zeros(ws, dtype=torch.uint8, device=device)
        self.ws_unmask = torch.zeros(B.bc_unmask_workspace_bytes(N * Rmax, V), dtype=torch.uint8, device=device)
        self.ws_verify = torch.zeros(B.bc_verify_workspace_bytes(N, Rmax, V), dtype=torch.uint8, device=device)
        self.scale = 1.0 / np.sqrt(D)
        # host staging through pinned memory
        pin = lambda n, dt: torch.zeros(n, dtype=dt).pin_memory()
        self.h_masked, self.h_tokens = pin(N * Rmax, torch.uint8), pin(N * Rmax, torch.int32)
        self.h_first, self.h_acc, self.h_bonus = pin(N, torch.int32), pin(N, torch.int32), pin(N, torch.int32)
        self.h_drafts = pin(N * Rmax, torch.int32)
        self.h_idx = {k: pin(N * Rmax, torch.int64) for k in ("draft", "verify")}
        self.d_idx = {k: torch.zeros(N * Rmax, dtype=torch.int64, device=device) for k in ("draft", "verify")}
        self.saved = {k: torch.zeros(N * Rmax, dtype=torch.float32, device=device) for k in ("draft", "verify")}
        self.trace, self.rounds = [], []
        self.result = None
        # the synthetic model's per-round draws, kept once drawn (a decode
        # repeated with the same agreement rate reads them from here); the
        # planted positions are kept on the device
        self._targets, self._plant_idx = {}, {}
        # the round's library calls, marshalled once per (block, active
        # rollouts, pool entry) and reissued; the private lengths are read
        # from this host array at each call
        self._calls = {}
        self._pl = np.zeros(N, np.int32)
        self._prefix_len = np.array([self.prefix], np.int32)

    def targets(self, b, r, s):
        """(verify argmax targets, drafts) [R_b] of rollout s in round r."""
        key = (b, r, s, self.p_agree)
        hit = self._targets.get(key)
        if hit is None:
            R = self.blocks[b]
            t = synth.round_targets(self.seed, self.V, R, 600 + b, r, s)
            hit = self._targets[key] = (t, synth.drafts_with_agreement(self.seed, t, self.p_agree, self.V,
                                                                       600 + b, r, s))
        return hit

    def host_logits(self, kind, b, r, active, base):
        """The round's float32 logits [len(active)][R_b][V] on the host, from
        the host copy ``base`` of the kind's clipped base (flat)."""
        R, V, n = self.blocks[b], self.V, len(active)
        x = base[: n * R * V].reshape(n, R, V).copy()
        for j, s in enumerate(active):
            t, d = self.targets(b, r, s)
            x[j, np.arange(R), t if kind == "verify" else d] = self.peak
        return x

    def host_qkv(self, b, r, pass_id):
        """float32 host arrays (q, k, v) of the pool entry round r reads."""
        (_, q), (_, k), (_, v) = synth.active_qkv(self.seed, self.N, self.blocks[b], self.Hq, self.Hkv, self.D,
                                                  self.dtype, 100 + b, pass_id, r % self.pool)
        return q, k, v

    def _plant(self, b, r, active):
        R, V, n = self.blocks[b], self.V, len(active)
        key = (b, r, tuple(active), self.p_agree)
        flat_idx = self._plant_idx.get(key)
        if flat_idx is None:
            flat_idx = {}
            for kind in ("draft", "verify"):
                x = np.empty(n * R, np.int64)
                for j, s in enumerate(active):
                    t, d = self.targets(b, r, s)
                    x[j * R:(j + 1) * R] = (j * R + np.arange(R)) * V + (t if kind == "verify" else d)
                flat_idx[kind] = torch.from_numpy(x).to(self.dev, non_blocking=False)
            self._plant_idx[key] = flat_idx
        self._planted = flat_idx
        for kind in ("draft", "verify"):
            idx = flat_idx[kind]
            flat = self.base[kind]
            torch.index_select(flat, 0, idx, out=self.saved[kind][: n * R])
            flat.index_fill_(0, idx, float(self.peak))

    def _restore(self, n_rows):
        for kind in ("draft", "verify"):
            self.base[kind].index_copy_(0, self._planted[kind], self.saved[kind][:n_rows])

    def _round_calls(self, b, n, r, priv, masked, tokens, first_d, out):
        """The round's four library calls for n active rollouts of block b,
        marshalled on first use and kept."""
        key = (b, n, r % self.pool)
        hit = self._calls.get(key)
        if hit is None:
            R, V = self.blocks[b], self.V
            qkv = [self.qkv[(b, r % self.pool, pass_id)] for pass_id in (0, 1)]
            pl = self._pl[:n]
            off = list(range(0, n * R + 1, R))
            draft, verify = (B.prepare_attn_step(self.shared, self._prefix_len, priv, pl, *(x[:n] for x in qkv[i]),
                                                 [0, R], mask, self.scale, out, self.ws_attn)
                             for i, mask in ((0, B.BC_MASK_BLOCK_BIDIR), (1, B.BC_MASK_BLOCK_CAUSAL)))
            dlg = self.base["draft"][: n * R * V].view(n * R, V)
            argmax = B.prepare_unmask_select(dlg, off, [B.BC_UNMASK_SEMI] * n, [1] * n, 0.0, masked, tokens, None,
                                             self.n_commit[:n], self.ws_unmask)
            vlg = self.base["verify"][: n * R * V].view(n, R, V)
            spec = B.prepare_spec_verify(vlg, tokens.view(n, R), None, first_d, self.accept_len[:n], self.bonus[:n],
                                         self.ws_verify)
            hit = self._calls[key] = (draft, argmax, verify, spec, qkv)
        return hit

    def run(self, stream=None, after_pass=None):
        """Decode the whole section for every rollout.  Returns the decoded
        tokens [N][sum(blocks)] (also in ``self.result``); ``self.trace``
        holds one dict per round (block, round, active, first, accept,
        bonus), ``self.rounds`` the rounds per block.  ``after_pass(b, r,
        pass_id, active, out)`` is called after each attention pass.  All
        device work is issued on ``stream`` (a torch stream, or None for the
        current one)."""
        if stream is None:
            return self._run(None, after_pass)
        with torch.cuda.stream(stream):
            return self._run(stream, after_pass)

    def _run(self, stream, after_pass):
        N, Hq, Hkv, D, V = self.N, self.Hq, self.Hkv, self.D, self.V
        self.priv_len[:] = 0
        result = np.full((N, self.cap), -1, np.int32)
        self.trace, self.rounds = [], []
        row0 = 0
        for b, R in enumerate(self.blocks):
            first = np.zeros(N, np.int64)
            verified = np.full((N, R), -1, np.int32)
            active, compacted = list(range(N)), None
            pl = int(self.priv_len[0])
            last_k = self.last_k[: N * Hkv * R * D].view(N, Hkv, R, D)
            last_v = self.last_v[: N * Hkv * R * D].view(N, Hkv, R, D)
            r = 0
            while active:
                n = len(active)
                if n == N:
                    priv = self.priv
                else:
                    if active != compacted and pl > 0:
                        idx = torch.tensor(active, dtype=torch.int64, device=self.dev)
                        for src, dst in ((self.priv.k, self.sub.k), (self.priv.v, self.sub.v)):
                            dst[:n, :, :pl] = src.index_select(0, idx)[:, :, :pl]
                    compacted = active
                    priv = B.KVCache(self.sub.k[:n], self.sub.v[:n])
                # the round's state: verified rows unmasked with their tokens
                fa = first[active]
                hm, ht = self.h_masked[: n * R].numpy(), self.h_tokens[: n * R].numpy()
                hm[:] = (np.arange(R)[None, :] >= fa[:, None]).ravel()
                ht[:] = verified[active].ravel()
                self.h_first[:n].numpy()[:] = fa
                masked, tokens, first_d = self.masked[: n * R], self.tokens[: n * R], self.first[:n]
                masked.copy_(self.h_masked[: n * R], non_blocking=True)
                tokens.copy_(self.h_tokens[: n * R], non_blocking=True)
                first_d.copy_(self.h_first[:n], non_blocking=True)
                self._plant(b, r, active)
                out = self.out[: n * R * Hq * D].view(n, R, Hq, D)
                self._pl[:n] = pl
                draft, argmax, verify, spec, qkv = self._round_calls(b, n, r, priv, masked, tokens, first_d, out)
                draft()
                if after_pass is not None:
                    after_pass(b, r, 0, list(active), out)
                argmax()
                verify()
                if after_pass is not None:
                    after_pass(b, r, 1, list(active), out)
                spec()
                self._restore(n * R)
                k, v = qkv[1][1][:n], qkv[1][2][:n]
                self.h_acc[:n].copy_(self.accept_len[:n], non_blocking=True)
                self.h_bonus[:n].copy_(self.bonus[:n], non_blocking=True)
                self.h_drafts[: n * R].copy_(tokens, non_blocking=True)
                torch.cuda.current_stream().synchronize()
                acc, bon = self.h_acc[:n].tolist(), self.h_bonus[:n].tolist()
                drafts = self.h_drafts[: n * R].numpy().reshape(n, R)
                self.trace.append(dict(block=b, round=r, active=list(active),
                                       first=[int(first[s]) for s in active], accept=acc, bonus=bon))
                # accepted drafts, then the bonus at the first mismatch
                A, Bo, act_arr = np.asarray(acc), np.asarray(bon), np.asarray(active)
                cols = np.arange(R)[None, :]
                take = (cols >= fa[:, None]) & (cols < (fa + A)[:, None])
                vs = verified[act_arr]
                vs[take] = drafts[take]
                hasb = Bo >= 0
                vs[np.nonzero(hasb)[0], (fa + A)[hasb]] = Bo[hasb]
                verified[act_arr] = vs
                nf = fa + A + hasb
                first[act_arr] = nf
                fin = nf >= R
                still = act_arr[~fin].tolist()
                done_slot, done_seq = np.nonzero(fin)[0].tolist(), act_arr[fin].tolist()
                if done_seq:
                    # the K/V of this (their last) verify pass are what they commit
                    js = torch.tensor(done_slot, dtype=torch.int64, device=self.dev)
                    ss = torch.tensor(done_seq, dtype=torch.int64, device=self.dev)
                    last_k.index_copy_(0, ss, k.index_select(0, js))
                    last_v.index_copy_(0, ss, v.index_select(0, js))
                active = still
                r += 1
            self.rounds.append(r)
            result[:, row0:row0 + R] = verified
            # every rollout holds pl private rows: one commit of all of them
            B.bc_kv_commit(self.priv, self.priv_len, B.BC_ALL_SEQ, pl, R, last_k, last_v, stream=stream)
            row0 += R
        self.result = result
        return result


class PipelinedDecode:
    """Pipelined parallel decoding (Fast-dVLA notes, key design 4 and its
    complete example) over the library calls.

    The output is a sequence of blocks decoded causally over a committed
    prefix, several at a time:
      * the first uncommitted block is fully active;
      * the block after an active one joins as semi-active (threshold-only
        commits) once its predecessor's completion ratio -- revealed tokens /
        block size, in double precision -- exceeds ``add`` (strictly), if
        fewer than ``window`` blocks are active; it becomes fully active
        (threshold plus at least ceil(remaining / n_div) per step) once the
        ratio exceeds ``act``;
      * every step runs one attention call over the committed cache with all
        active blocks (bidirectional inside a block, causal across) and one
        unmask call with a mode per block;
      * a block whose tokens are all revealed is committed to the cache, with
        the K/V of its last step, as soon as every earlier block is: strictly
        in order, right after that step.
    The schedule is the library's native state machine (``bc_pipeline_*``,
    host code): it needs each step's commit counts, so the host reads them
    back after every step; the schedule is data-dependent and host-driven.

    Block b's synthetic model outputs at its s-th active step are seeded
    draws: logits (``logits_for``) and the rows' Q/K/V (``qkv_for``)."""

    def __init__(self, preset=None, seed=0, device="cuda:0", add=0.5, act=0.9, tau=0.5, n_div=4,
                 window=None, planted_frac=0.2):
        p = dict(preset or synth.PRESETS["pipelined_625"])
        self.Hq, self.Hkv, self.D = p["n_q_heads"], p["n_kv_heads"], p["head_dim"]
        self.dtype, self.V, self.sigma = p["dtype"], p["vocab"], p["sigma"]
        self.blocks = list(p["blocks"])
        self.prefix = p["prefix"]
        self.window = int(window or p.get("window", 3))
        self.add, self.act, self.tau, self.n_div = float(add), float(act), float(tau), int(n_div)
        if self.window < 1 or self.n_div < 1:
            raise ValueError("window and n_div must be at least 1")
        self.seed, self.planted_frac, self.dev = seed, planted_frac, device
        nb = len(self.blocks)
        self.cap = self.prefix + sum(self.blocks)
        self.row0 = [0] + [int(x) for x in np.cumsum(self.blocks)]
        (k, v), _ = synth.kv_cache(seed, 1, self.Hkv, self.cap, self.D, [self.prefix], self.dtype)
        self.cache = B.KVCache(k.to(device), v.to(device))
        n_out = sum(self.blocks)
        self.masked = torch.ones(n_out, dtype=torch.uint8, device=device)
        self.tokens = torch.full((n_out,), -1, dtype=torch.int32, device=device)
        self.n_commit = torch.zeros(self.window, dtype=torch.int32, device=device)
        # active sets are runs of at most `window` consecutive blocks
        runs = [self.blocks[i:i + w] for i in range(nb) for w in range(1, self.window + 1) if i + w <= nb]
        ws = 0
        for r in runs:
            off = [0] + [int(x) for x in np.cumsum(r)]
            ws = max(ws, B.bc_attn_workspace_bytes(self.cache, None, (1, off[-1], self.Hq, self.D), off))
        rmax = max(sum(r) for r in runs)
        self.ws_attn = torch.zeros(ws, dtype=torch.uint8, device=device)
        self.ws_unmask = torch.zeros(B.bc_unmask_workspace_bytes(rmax, self.V), dtype=torch.uint8, device=device)
        self.out = torch.empty((1, rmax, self.Hq, self.D), dtype=synth.torch_dtype(self.dtype), device=device)
        self.scale = 1.0 / np.sqrt(self.D)
        self.trace = []
        self.length = np.array([self.prefix], np.int32)
        self.keep_inputs = False
        self._resident = {}
        self._calls = {}
        self._native = {}
        self._dev = None
        self._dev_graph = None
        self._dev_max_local = 0
        # the commit counts come back through pinned host memory
        self.n_commit_host = torch.zeros(self.window, dtype=torch.int32).pin_memory()

    def logits_for(self, b, s):
        x = synth.logits(self.seed, self.blocks[b], self.V, self.sigma, 700 + b, s)
        if self.planted_frac:
            synth.plant_peaks(x, self.seed, self.planted_frac, 12.0, 700 + b, s)
        return x

    def qkv_for(self, b, s):
        """((q, q32), (k, k32), (v, v32)) of block b at its s-th active step:
        q [1][rows][Hq][D], k / v [1][Hkv][rows][D]."""
        return synth.active_qkv(self.seed, 1, self.blocks[b], self.Hq, self.Hkv, self.D, self.dtype, 800 + b, s)

    def _step_inputs(self, active, steps):
        """Device q, k, v, logits of one step (the active blocks' rows in
        order).  With keep_inputs set they stay resident, keyed by the step's
        (blocks, local steps): the schedule is deterministic, so a second run
        finds every step's inputs already on the device."""
        key = (tuple(active), tuple(steps))
        hit = self._resident.get(key)
        if hit is not None:
            return hit
        qkv = [self.qkv_for(b, st) for b, st in zip(active, steps)]
        x = (torch.cat([t[0][0] for t in qkv], dim=1).to(self.dev),
             torch.cat([t[1][0] for t in qkv], dim=2).to(self.dev),
             torch.cat([t[2][0] for t in qkv], dim=2).to(self.dev),
             torch.from_numpy(np.concatenate([self.logits_for(b, st) for b, st in zip(active, steps)])).to(self.dev),
             [(t[1][0][0].to(self.dev), t[2][0][0].to(self.dev)) for t in qkv])   # per block [Hkv][rows][D]
        if self.keep_inputs:
            self._resident[key] = x
        return x

    def run(self, stream=None, after_attn=None):
        """Decode every block; returns the number of steps (the trace of each
        step is in ``self.trace``, tokens in ``self.tokens``).
        after_attn(step, active, local_steps, length, out) is called after each
        step's attention call (``out`` is the view it wrote).  Every device
        operation, torch's own fills and copies included, is issued on
        ``stream`` (a torch stream, or None for the current one)."""
        if stream is None:
            return self._run(None, after_attn)
        with torch.cuda.stream(stream):
            return self._run(stream, after_attn)

    def run_native(self, stream=None, after_attn=None):
        """The same decode with the step loop inside the library
        (``bc_pipeline_decode``): the schedule, the calls, the commits and
        the read-back of each step's commit counts (polled in mapped host
        memory, no stream synchronisation) run natively; Python only hands
        over each step's model outputs through a callback.  Same arguments
        and results as ``run``."""
        if stream is None:
            return self._run_native(None, after_attn)
        with torch.cuda.stream(stream):
            return self._run_native(stream, after_attn)

    def _native_inputs(self, active, steps):
        key = (tuple(active), tuple(steps))
        hit = self._native.get(key)
        if hit is not None:
            return hit
        q, k, v, lg, blk_kv = self._step_inputs(active, steps)
        st = B.BcStepInputs()
        st.q, st.k, st.v, st.logits = q.data_ptr(), k.data_ptr(), v.data_ptr(), lg.data_ptr()
        for j, (bk, bv) in enumerate(blk_kv):
            st.blk_k[j], st.blk_v[j] = bk.data_ptr(), bv.data_ptr()
        hit = (st, (q, k, v, lg, blk_kv))
        if self.keep_inputs:
            self._native[key] = hit
        return hit

    def _run_native(self, stream, after_attn):
        sched = B.Pipeline(self.blocks, self.window, self.add, self.act, self.n_div)
        self.length[0] = self.prefix
        self.masked.fill_(1)
        self.tokens.fill_(-1)
        live = []   # without resident inputs: the last steps' tensors stay referenced

        def inputs(step, active, steps):
            st, tensors = self._native_inputs(active, steps)
            live.append(tensors)
            del live[:-2]
            return st

        hook = None
        if after_attn is not None:
            def hook(step, active, steps, length, _out):
                after_attn(step, active, steps, length, self.out[:, :sum(self.blocks[b] for b in active)])
        try:
            n, self.trace = sched.decode(self.cache, self.length, self.Hq, self.V, self.scale, self.tau, self.masked,
                                         self.tokens, self.out, self.ws_attn, self.ws_unmask, inputs, hook,
                                         max_steps=sum(self.blocks) + len(self.blocks), stream=stream)
        finally:
            sched.close()
        return n

    def run_device(self, stream=None, max_local=None, steps_per_graph=8, after_step=None):
        """The same decode with the schedule on the device
        (``bc_pipeline_dev_*``): each step is the model's stand-in (a copy of
        the planned blocks' seeded outputs into fixed step buffers), the
        attention, the unmask and the schedule kernel, and no step reads
        anything back.  Runs of ``steps_per_graph`` steps are captured once
        in a graph and replayed, one replay queued ahead, until the schedule
        reports the end (steps after it do nothing).  ``max_local`` bounds the local steps whose
        outputs are staged (default: from the previous ``run``'s trace, one
        more than any block's); a step past it stops the decode with an
        error.  With ``after_step(k, active, local_steps, length, out)`` the
        steps run one by one, without graphs, and the hook sees each step's
        attention output.  Same results as ``run``, except that the
        attention follows the widest step's split plan."""
        own = stream is None
        if own:   # graphs are not captured on the legacy default stream
            if getattr(self, "_dev_stream", None) is None:
                self._dev_stream = torch.cuda.Stream(device=self.dev)
            stream = self._dev_stream
            stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            n = self._run_device(stream, max_local, steps_per_graph, after_step)
        if own:
            torch.cuda.current_stream().wait_stream(stream)
        return n

    def _device_setup(self, max_local):
        if max_local is None:
            if not self.trace:
                raise ValueError("max_local: run() first, or pass the bound")
            max_local = 1 + max(sum(1 for st in self.trace if b in st["active"]) for b in range(len(self.blocks)))
        if self._dev is not None and self._dev_max_local >= max_local:
            return
        self._dev = None
        self._dev_graph = None
        R = max(sum(self.blocks[i:i + self.window]) for i in range(len(self.blocks)))
        dt = synth.torch_dtype(self.dtype)
        self.step_q = torch.zeros((1, R, self.Hq, self.D), dtype=dt, device=self.dev)
        self.step_k = torch.zeros((1, self.Hkv, R, self.D), dtype=dt, device=self.dev)
        self.step_v = torch.zeros((1, self.Hkv, R, self.D), dtype=dt, device=self.dev)
        self.step_logits = torch.zeros((R, self.V), dtype=torch.float32, device=self.dev)
        self.step_out = torch.zeros((1, R, self.Hq, self.D), dtype=dt, device=self.dev)
        # the seeded model outputs of every (block, local step) below the bound
        nb = len(self.blocks)
        entries = (B.BcStepBlock * (nb * max_local))()
        staged = []
        for b in range(nb):
            for st in range(max_local):
                (q, _), (k, _), (v, _) = self.qkv_for(b, st)
                x = (q.to(self.dev).contiguous(), k.to(self.dev).contiguous(), v.to(self.dev).contiguous(),
                     torch.from_numpy(self.logits_for(b, st)).to(self.dev))
                staged.append(x)
                e = entries[b * max_local + st]
                e.q, e.k, e.v, e.logits = (t.data_ptr() for t in x)
        self._dev_staged = staged
        self._dev_table = torch.frombuffer(bytearray(bytes(entries)), dtype=torch.uint8).to(self.dev)
        self._dev = B.DevicePipeline(self.blocks, self.window, self.add, self.act, self.n_div, self.cache, self.prefix,
                                     self.Hq, self.V, self.scale, self.tau, self.masked, self.tokens, self.step_q,
                                     self.step_k, self.step_v, self.step_logits, self.step_out,
                                     sum(self.blocks) + nb)
        self._dev_max_local = max_local

    def _run_device(self, stream, max_local, steps_per_graph, after_step):
        self._device_setup(max_local)
        dev = self._dev
        s = torch.cuda.current_stream()
        self.masked.fill_(1)
        self.tokens.fill_(-1)
        dev.reset(s)
        if after_step is None:
            if self._dev_graph is None or self._dev_graph[1] != steps_per_graph:
                s.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=s):
                    for _ in range(steps_per_graph):
                        dev.replay(self._dev_table, self._dev_max_local, s)
                        dev.step(s)
                self._dev_graph = (g, steps_per_graph)
                # capture enqueued nothing: start again
                self.masked.fill_(1)
                self.tokens.fill_(-1)
                dev.reset(s)
            # one replay always queued behind the one being waited on, so
            # the GPU never idles on the host's check; at most that one runs
            # past the end, as steps that do nothing
            g = self._dev_graph[0]
            pending = []
            for _ in range(2):
                g.replay()
                pending.append(torch.cuda.Event())
                pending[-1].record(s)
            while True:
                pending.pop(0).synchronize()
                if dev.status()[0]:
                    break
                g.replay()
                pending.append(torch.cuda.Event())
                pending[-1].record(s)
            s.synchronize()
            finished, n, length, err = dev.status()
        else:
            k = 0
            while True:
                plan = dev.read_plan()   # synchronises
                if plan.n == 0:
                    break
                dev.replay(self._dev_table, self._dev_max_local, s)
                dev.step(s)
                s.synchronize()
                rows = plan.rows
                after_step(k, list(plan.active[:plan.n]), list(plan.local_step[:plan.n]), plan.len,
                           self.step_out[:, :rows])
                k += 1
            finished, n, length, err = dev.status()
        if err:
            raise RuntimeError("device pipelined decode stopped: error %d" % err)
        self.trace = dev.trace()
        self.length[0] = length
        return n

    def _run(self, stream, after_attn):
        sched = B.Pipeline(self.blocks, self.window, self.add, self.act, self.n_div)
        self.length[0] = self.prefix
        self.masked.fill_(1)
        self.tokens.fill_(-1)
        self.trace = []
        while True:
            plan = sched.plan()
            if plan is None:
                break
            active, steps, modes, divs, off, r0 = plan
            rows = off[-1]
            key = (tuple(active), tuple(steps), tuple(modes), B._stream(stream))
            calls = self._calls.get(key)
            if calls is None:
                # the step's two library calls, marshalled once (with
                # resident inputs they are kept and reissued on later runs)
                q, k, v, lg, blk_kv = self._step_inputs(active, steps)
                out = self.out[:, :rows]
                nc = self.n_commit[:len(active)]
                calls = (B.prepare_attn_step(self.cache, self.length, None, None, q, k, v, off,
                                             B.BC_MASK_BLOCK_BIDIR, self.scale, out, self.ws_attn, stream=stream),
                         B.prepare_unmask_select(lg, off, modes, divs, self.tau, self.masked[r0:r0 + rows],
                                                 self.tokens[r0:r0 + rows], None, nc, self.ws_unmask, stream=stream),
                         blk_kv, out, nc)
                if self.keep_inputs:
                    self._calls[key] = calls
            attn, unmask, blk_kv, out, nc = calls
            attn()
            if after_attn is not None:
                after_attn(len(self.trace), list(active), steps, int(self.length[0]), out)
            unmask()
            # the next plan depends on the counts: copy them to pinned memory
            # and wait for the stream
            host = self.n_commit_host[:len(active)]
            host.copy_(nc, non_blocking=True)
            torch.cuda.current_stream().synchronize()
            counts = [int(x) for x in host.tolist()]
            done = sched.report(counts)
            for b in done:                          # in order, with the K/V of the block's last step
                blk_k, blk_v = blk_kv[active.index(b)]
                B.bc_kv_commit(self.cache, self.length, 0, int(self.length[0]), self.blocks[b], blk_k, blk_v,
                               stream=stream)
            self.trace.append(dict(active=list(active),
                                   modes=["full" if m == B.BC_UNMASK_FULL else "semi" for m in modes],
                                   n_commit=counts, committed=list(done)))
        sched.close()
        return len(self.trace)
