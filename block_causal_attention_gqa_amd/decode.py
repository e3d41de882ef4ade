"""Host decode schedules driving the C-ABI calls.

Every step of the path runs in the HIP kernels behind ``binding``; this
module only owns device buffers and issues the calls in the order the pages
describe:

* ``SectionDecode`` -- Section Diffusion (Fast-dDrive method summary,
  sec. 3.2): output blocks are decoded in causal order over a committed
  prefix; each block takes a fixed number of denoise steps (attention, then
  confidence unmask with n = steps left), and its K/V are committed to the
  cache when it completes.  Also the large-block decode at batch > 1 (one
  attention call covers every sequence; the unmask call sees one block per
  sequence).
* ``ForkVerify`` -- shared-prefix fork with scaffold speculative decoding
  (method summary sec. 3.2 - 3.3): N rollouts share one prefix cache; per
  trajectory block and round, a bidirectional draft pass, a draft argmax
  (threshold 0 reveals every masked row), a causal verify pass and the
  verify call.

The model between attention and logits is not part of this library:
attention outputs are produced and discarded, logits and the active rows'
Q/K/V are seeded synthetic tensors made up-front and resident on the GPU.
"""

import numpy as np
import torch

from . import binding as B
from . import synth


class SectionDecode:
    def __init__(self, preset, seed=0, n_seq=None, device="cuda:0", logits_pool=None,
                 planted_frac=0.0, planted_delta=12.0):
        p = dict(preset)
        self.p = p
        self.S = n_seq or p.get("n_seq", 1)
        self.Hq, self.Hkv, self.D = p["n_q_heads"], p["n_kv_heads"], p["head_dim"]
        self.dtype = p["dtype"]
        self.blocks = list(p["blocks"])
        self.steps = p["steps"]
        self.V, self.sigma, self.tau = p["vocab"], p["sigma"], p["threshold"]
        self.prefix = p["prefix"]
        self.cap = self.prefix + sum(self.blocks)
        self.dev = device
        S, Hkv, D = self.S, self.Hkv, self.D
        tdt = synth.torch_dtype(self.dtype)
        (k, v), _ = synth.kv_cache(seed, S, Hkv, self.cap, D, [self.prefix] * S, self.dtype)
        self.cache = B.KVCache(k.to(device), v.to(device))
        self.len0 = np.full(S, self.prefix, np.int32)
        # per (block, step) active rows and logits, resident on the device;
        # with logits_pool = k, k distinct logits tensors are cycled instead
        bmax = max(self.blocks)
        self.qkv = []
        for b, bs in enumerate(self.blocks):
            row = []
            for st in range(self.steps):
                (qt, _), (kt, _), (vt, _) = synth.active_qkv(seed, S, bs, self.Hq, Hkv, D, self.dtype, b, st)
                row.append((qt.to(device), kt.to(device), vt.to(device)))
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
        self.out = {bs: torch.empty((S, bs, self.Hq, D), dtype=tdt, device=device) for bs in set(self.blocks)}
        self.masked = torch.ones(S * sum(self.blocks), dtype=torch.uint8, device=device)
        self.tokens = torch.full((S * sum(self.blocks),), -1, dtype=torch.int32, device=device)
        self.conf = torch.empty(S * bmax, dtype=torch.float32, device=device)
        self.n_commit = torch.zeros(self.S, dtype=torch.int32, device=device)
        self.ws_attn = torch.zeros(max(B.bc_attn_workspace_bytes(self.cache, None, (S, bs, self.Hq, D), [0, bs])
                                       for bs in set(self.blocks)), dtype=torch.uint8, device=device)
        self.ws_unmask = torch.zeros(B.bc_unmask_workspace_bytes(S * bmax, self.V), dtype=torch.uint8,
                                     device=device)
        self.scale = 1.0 / np.sqrt(D)
        self.hooks = None   # optional callables around each call: hooks(kind, "pre"/"post")

    @property
    def tokens_per_decode(self):
        return self.S * sum(self.blocks)

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
        off = 0
        for b, bs in enumerate(self.blocks):
            masked = self.masked[S * off: S * (off + bs)]
            tokens = self.tokens[S * off: S * (off + bs)]
            masked.fill_(1)
            blk_rows = list(range(0, S * bs + 1, bs))
            out = self.out[bs]
            for st in range(self.steps):
                q, k, v = self.qkv[b][st]
                self._hook("attn", "pre")
                B.bc_attn_step(self.cache, length, None, None, q, k, v, [0, bs], B.BC_MASK_BLOCK_BIDIR,
                               self.scale, out, self.ws_attn, stream=stream)
                self._hook("attn", "post")
                self._hook("unmask", "pre")
                B.bc_unmask_select(self.logits[b][st], blk_rows, [B.BC_UNMASK_FULL] * S,
                                   [self.steps - st] * S, self.tau, masked, tokens, self.conf[: S * bs],
                                   self.n_commit[:S], self.ws_unmask, stream=stream)
                self._hook("unmask", "post")
            q, k, v = self.qkv[b][self.steps - 1]
            self._hook("commit", "pre")
            for s in range(S):
                B.bc_kv_commit(self.cache, length, s, int(length[s]), bs, k[s], v[s], stream=stream)
            self._hook("commit", "post")
            off += bs


class ForkVerify:
    """One round of the shared-prefix fork with scaffold speculative
    decoding for one trajectory block (Fast-dDrive method summary sec. 3.2,
    3.3): N rollouts share one prefix cache and keep their earlier trajectory
    blocks in private caches.  A round is

      1. draft pass: bidirectional attention of the block's rows;
      2. draft argmax: an unmask with threshold 0 and SEMI mode reveals every
         masked row, token = argmax of its draft logits;
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
        g = synth.rng(seed, "misc", 400 + block)
        self.fixed = torch.from_numpy((g.random((N, R)) < scaffold_frac).astype(np.uint8)).to(device)
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
        return dict(pk=pk, pv=pv, vk=vk, vv=vv, qkv=qkv, noise=noise,
                    draft_logits=synth.logits(seed, N * R, self.V, self.sigma, 200 + block),
                    verify_logits=synth.logits(seed, N * R, self.V, self.sigma, 300 + block).reshape(N, R, self.V),
                    fixed=self.fixed.cpu().numpy())

    def attention(self, pass_id, stream=None):
        q, k, v = self.qkv[pass_id]
        mask = B.BC_MASK_BLOCK_BIDIR if pass_id == 0 else B.BC_MASK_BLOCK_CAUSAL
        B.bc_attn_step(self.shared, [self.prefix], self.priv, self.priv_len, q, k, v, [0, self.R], mask,
                       self.scale, self.out, self.ws_attn, stream=stream)

    def draft_argmax(self, stream=None):
        self.masked.fill_(1)
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
