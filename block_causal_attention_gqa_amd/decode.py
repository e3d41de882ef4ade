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
