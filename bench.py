#!/usr/bin/env python3
"""Throughput of the block-causal denoising step on one MI355X.

Workload: the Fast-dDrive-shaped section decode at batch 1 -- 16 query / 2
KV heads, head_dim 128, bf16 K/V, a 3072-token committed prefix, editable
sections of 12 / 192 / 6 / 70 tokens cut into blocks of 32 (11 blocks, 280
tokens), 8 denoise steps per block, each step = block-causal attention over
the cache + confidence unmask over fp32 logits [b x 151936] ~ N(0, 4^2) with
threshold 0.9 and n = steps left; the block's K/V are committed when it
completes.  All inputs are seeded synthetic tensors resident in HBM before
timing starts.

One bench step = one whole section decode (88 denoise steps, 11 commits),
replayed as a captured HIP graph.  value = decoded tokens / s.

Prints ONE JSON line.  Options: --steps K --warmup W (timed decodes /
untimed decodes), --mode graph|eager, --no-cpu-baseline.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "denoise-step ms + decoded tok/s at bs1 B=32; attn HBM TB/s vs roofline"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--mode", choices=["graph", "eager"], default="graph")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the oracle decode until this much CPU time is spent")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="for hardware-counter runs: issue one decode's attention-partial launches and a "
                         "256 MiB device copy (the counters' calibration), print one JSON line, exit")
    ap.add_argument("--fork-pass", action="store_true",
                    help="for profiler runs: issue the N = 64 fork round's two attention calls (draft pass, "
                         "verify pass) 10 times each, print one JSON line, exit")
    ap.add_argument("--verify-pass", action="store_true",
                    help="for profiler runs: issue the N = 64 fork round's verify scan (greedy, then sampled "
                         "with Gumbel noise) 10 times each and a 256 MiB device copy (the counters' "
                         "calibration), print one JSON line, exit")
    ap.add_argument("--batch-pass", action="store_true",
                    help="for profiler runs: issue the large-block attention call at batch 16 (32q/8kv, a "
                         "32-row block over a 2176-key prefix) 10 times over 5 distinct caches (765 MB, more "
                         "than the MALL holds) and a 256 MiB device copy (the counters' calibration), print one "
                         "JSON line, exit")
    ap.add_argument("--no-legs", action="store_true",
                    help="skip the secondary measurements (fork round, batch-16 attention, verify scan)")
    return ap.parse_args()


def attn_bytes_flops(prefix_len, R, Hq, Hkv, D, elem=2):
    """Algorithmic bytes / flops of one BIDIR single-block attention call."""
    L = prefix_len + R
    kv = 2 * Hkv * L * D * elem
    qo = 2 * R * Hq * D * elem
    flops = 4 * D * Hq * R * L
    return kv + qo, flops


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    import torch
    from block_causal_attention_gqa_amd import binding as B
    from block_causal_attention_gqa_amd import decode, synth

    B.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    if args.fork_pass:
        fork_pass()
        return
    if args.verify_pass:
        verify_pass()
        return
    if args.batch_pass:
        batch_pass()
        return
    preset = synth.PRESETS["section"]
    t0 = time.time()
    dec = decode.SectionDecode(preset, seed=args.seed, device=dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t0
    if args.pmc_pass:
        pmc_pass(dec)
        return

    stream = torch.cuda.Stream()
    graph = None
    with torch.cuda.stream(stream):
        dec.run()            # eager once before capture (library + torch warm)
    torch.cuda.synchronize()
    if args.mode == "graph":
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            dec.run()
        torch.cuda.synchronize()

    def one():
        # graph replays and eager calls both go to `stream`, where the events are
        with torch.cuda.stream(stream):
            if graph is not None:
                graph.replay()
            else:
                dec.run()

    for _ in range(args.warmup):
        one()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        one()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = ev0.elapsed_time(ev1)
    ms_per_step = ms_total / args.steps

    # sanity: the decode finished every block
    assert int(dec.masked.sum().item()) == 0, "decode left masked rows"
    assert int((dec.tokens < 0).sum().item()) == 0
    # what the last timed replay left, for the oracle check
    timed_out = {"tokens": dec.tokens.cpu().numpy(), "masked": dec.masked.cpu().numpy(),
                 "cache_k": dec.cache.k[0].float().cpu().numpy(), "cache_v": dec.cache.v[0].float().cpu().numpy()}

    # the same decode issued call by call from the host (no graph), for the
    # graph's gain: host marshalling and launch per call sit between kernels
    graph_gain = None
    if graph is not None:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(3):
                dec.run()
            e1.record(stream)
        torch.cuda.synchronize()
        eager_ms = e0.elapsed_time(e1) / 3
        graph_gain = {"graph_ms": round(ms_per_step, 4), "eager_ms": round(eager_ms, 4),
                      "speedup": round(eager_ms / ms_per_step, 2)}

    # ---- per-kernel launch duration.  The decode is issued once more
    # through the sub-step entry points, saving the masked rows each scan
    # sees; then every step's launches of one kernel are captured back to
    # back in a graph of their own and replayed between two HIP events on
    # that graph's stream: total / launches is the average launch duration,
    # with no host gaps and no event between launches.
    masked_before = []
    call_args = []
    length = dec.len0.copy()
    off = 0
    with torch.cuda.stream(stream):
        for b, bs in enumerate(dec.blocks):
            masked = dec.masked[off: off + bs]
            tokens = dec.tokens[off: off + bs]
            masked.fill_(1)
            for st in range(dec.steps):
                q, k, v = dec.qkv[b][st]
                a_args = (dec.cache, length.copy(), None, None, q, k, v, [0, bs], B.BC_MASK_BLOCK_BIDIR,
                          dec.scale, dec.out[bs], dec.ws_attn)
                B.bc_attn_partial(*a_args, stream=stream)
                B.bc_attn_combine(*a_args, stream=stream)
                masked_before.append(masked.clone())
                lg = dec.logits[b][st]
                B.bc_vocab_scan(lg, masked, True, dec.ws_unmask, stream=stream)
                B.bc_unmask_decide(lg, [0, bs], [B.BC_UNMASK_FULL], [dec.steps - st], dec.tau, masked, tokens,
                                   dec.conf[:bs], dec.n_commit[:1], dec.ws_unmask, stream=stream)
                call_args.append((a_args, lg))
            q, k, v = dec.qkv[b][dec.steps - 1]
            B.bc_kv_commit(dec.cache, length, 0, int(length[0]), bs, k[0], v[0], stream=stream)
            off += bs
    torch.cuda.synchronize()
    assert int(dec.masked.sum().item()) == 0, "sub-step decode left masked rows"
    masked_rows = [int(m.sum().item()) for m in masked_before]

    def per_launch_us(issue, reps=10):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            issue()
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=stream):
                issue()
            g.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * len(call_args))

    avg = {
        "attn_partial": per_launch_us(lambda: [B.bc_attn_partial(*a, stream=stream) for a, _ in call_args]),
        "attn_combine": per_launch_us(lambda: [B.bc_attn_combine(*a, stream=stream) for a, _ in call_args]),
        # the whole call (partial, then combine) back to back: unlike the sum of
        # the two above, it includes the combine reading partials just written
        "attn_call": per_launch_us(lambda: [B.bc_attn_step(*a, stream=stream) for a, _ in call_args]),
        "vocab_scan": per_launch_us(lambda: [B.bc_vocab_scan(lg, m, True, dec.ws_unmask, stream=stream)
                                             for (_, lg), m in zip(call_args, masked_before)]),
    }

    # algorithmic work
    Hq, Hkv, D, V = dec.Hq, dec.Hkv, dec.D, dec.V
    attn_bytes, attn_flops, partial_bytes = 0, 0, 0
    length = dec.prefix
    for bs in dec.blocks:
        for _ in range(dec.steps):
            b_, f_ = attn_bytes_flops(length, bs, Hq, Hkv, D)
            attn_bytes += b_
            attn_flops += f_
            partial_bytes += b_ - bs * Hq * D * 2       # K/V and Q; the output is the combine's
        length += bs
    n_attn = len(call_args)
    attn_us = avg["attn_partial"] + avg["attn_combine"]
    attn_gbs = attn_bytes / n_attn / (attn_us * 1e-6) / 1e9
    attn_tflops = attn_flops / n_attn / (attn_us * 1e-6) / 1e12
    scan_bytes = sum(4 * V * r for r in masked_rows)
    n_scan = len(masked_rows)
    scan_gbs = scan_bytes / n_scan / (avg["vocab_scan"] * 1e-6) / 1e9
    tot = {k: v * n_attn for k, v in avg.items() if k != "attn_call"}
    dominant = max(("attn_partial", "vocab_scan"), key=tot.get)
    if dominant == "vocab_scan":
        roof = {"kernel": "scan_kernel (bc_vocab_scan: per-row max/argmax/exp-sum over the vocabulary)",
                "bound": "hbm", "achieved": round(scan_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(scan_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                "bytes_per_launch": scan_bytes / n_scan, "avg_launch_us": round(avg["vocab_scan"], 3)}
    else:
        pgbs = partial_bytes / n_attn / (avg["attn_partial"] * 1e-6) / 1e9
        roof = {"kernel": "attn_partial_bf16_kernel (bc_attn_partial: block-causal GQA attention, split-KV)",
                "bound": "hbm", "achieved": round(pgbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(pgbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                "bytes_per_launch": partial_bytes / n_attn, "avg_launch_us": round(avg["attn_partial"], 3)}
    kernel_us = {k: round(v, 3) for k, v in avg.items()}
    cold = cache_states(stream, dec, call_args, masked_before)

    tokens = dec.tokens_per_decode
    value = tokens * args.steps / (ms_total * 1e-3)
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 K/V/Q, N(0,4^2) fp32 logits; no model weights)",
        "config": {"workload": "section_decode bs1 B=32: 16q/2kv heads, head_dim 128, prefix 3072, "
                               "blocks 12/32x6/6/32/32/6, 8 denoise steps/block, vocab 151936",
                   "global_batch": 1, "seq_len": dec.prefix + sum(dec.blocks), "parallelism": "none (1 GPU)",
                   "mode": args.mode},
        "denoise_step_ms": round(ms_per_step / dec.denoise_steps, 5),
        "graph_vs_eager": graph_gain,
        "attn": {"avg_us": round(attn_us, 3), "call_us_back_to_back": round(avg["attn_call"], 3),
                 "TB_s_call": round(attn_bytes / n_attn / avg["attn_call"] / 1e6, 4),
                 "TB_s": round(attn_gbs / 1e3, 4),
                 "TFLOP_s": round(attn_tflops, 3), "hbm_frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                 "mfma_frac": round(attn_tflops / BF16_PEAK_TFLOPS, 5),
                 "bytes_per_call": attn_bytes / n_attn, "flops_per_call": attn_flops / n_attn},
        "unmask": {"scan_us": round(avg["vocab_scan"], 3), "scan_GB_s": round(scan_gbs, 1),
                   "avg_masked_rows": float(np.mean(masked_rows))},
        "kernel_avg_us": kernel_us,
        "cache_states": cold,
        "roofline": roof,
        "wall_s_timed": round(wall, 4),
        "setup_s": round(setup_s, 2),
    }

    if not args.no_legs:
        result["legs"] = legs(stream)
    if not args.no_cpu_baseline:
        result["cpu_baseline"], result["oracle_check"] = cpu_baseline(dec, args, timed_out)
    print(json.dumps(result), flush=True)


TRAFFIC_SUMMARY = "profiles/attn_partial_section_decode_traffic.md"


def cache_states(stream, dec, call_args, masked_before, reps=20, replays=5):
    """Cold and warm call times at the bs1 shape: the attention call
    (partial + combine) and the unmask select of the first denoise step of
    the first 32-row block.  One graph holds reps repetitions of [a flush,
    the call], another the same flushes alone; the call time is their
    difference / reps.  Cold dirty: the flush writes 512 MiB (the 256 MB
    MALL and the L2 hold none of the call's data and are full of dirty
    lines); cold clean: the flush reads 512 MiB (clean lines).  Warm: the
    same with a GPU spin that touches no memory in place of the flush (the
    call's data stay where the previous call left them).  Median over the
    replays."""
    import torch
    from block_causal_attention_gqa_amd import binding as B
    b = next(i for i, bs in enumerate(dec.blocks) if bs == 32)
    off, bs = sum(dec.blocks[:b]), dec.blocks[b]
    i = b * dec.steps
    a_args, lg = call_args[i]
    masked, tokens = dec.masked[off: off + bs], dec.tokens[off: off + bs]
    saved = masked_before[i]
    flush = make_flush(dec.masked.device)

    def attn():
        B.bc_attn_step(*a_args, stream=stream)

    def unmask():
        masked.copy_(saved)
        B.bc_unmask_select(lg, [0, bs], [B.BC_UNMASK_FULL], [dec.steps], dec.tau, masked, tokens, dec.conf[:bs],
                           dec.n_commit[:1], dec.ws_unmask, stream=stream)

    def restore():
        masked.copy_(saved)

    def pre(state):
        if state == "warm":
            torch.cuda._sleep(100000)
        else:
            flush[state]()

    def graph_ms(body):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            body()
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=stream):
                body()
            ts = []
            for _ in range(replays):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                g.replay()
                e1.record(stream)
                ts.append((e0, e1))
        torch.cuda.synchronize()
        return float(np.median([e0.elapsed_time(e1) for e0, e1 in ts]))

    out = {"shape": "bs1, 32-row block over a %d-key prefix, vocab %d, %d masked rows"
                    % (int(a_args[1][0]), dec.V, int(saved.sum().item())),
           "flush_bytes": flush["bytes"], "reps_per_graph": reps}
    for name, fn, base in (("attn_step_us", attn, lambda: None), ("unmask_select_us", unmask, restore)):
        out[name] = {}
        for state in ("cold_dirty", "cold_clean", "warm"):
            def with_call():
                for _ in range(reps):
                    pre(state.replace("cold_", ""))
                    fn()

            def without():
                for _ in range(reps):
                    pre(state.replace("cold_", ""))
                    base()
            out[name][state] = round((graph_ms(with_call) - graph_ms(without)) * 1e3 / reps, 3)
    masked.zero_()
    b_, _ = attn_bytes_flops(int(a_args[1][0]), bs, dec.Hq, dec.Hkv, dec.D)
    out["attn_TB_s"] = {k: round(b_ / (v * 1e-6) / 1e12, 4) for k, v in out["attn_step_us"].items()}
    return out


def measured_traffic():
    """HBM bytes per attn_partial launch from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, calibrated), or None when the attention
    sources changed since the counters were taken."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    try:
        text = open(os.path.join(root, TRAFFIC_SUMMARY)).read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if ":" in line and line.split(":", 1)[0] in ("traffic_bytes_per_launch", "source_sha256", "sources"):
            k, v = line.split(":", 1)
            fields[k] = v.strip()
    if not {"traffic_bytes_per_launch", "source_sha256", "sources"} <= fields.keys():
        return None
    h = hashlib.sha256()
    for f in fields["sources"].split(", "):
        h.update(open(os.path.join(root, f), "rb").read())
    if h.hexdigest() != fields["source_sha256"]:
        return None
    return float(fields["traffic_bytes_per_launch"])


def fork_pass(N=64, reps=10):
    """The shared-prefix fork round's attention calls at N rollouts (3282
    shared keys, 24 rows x 16 heads per rollout), each pass issued reps
    times after one warm call, for kernel traces and MFMA counters."""
    import torch
    from block_causal_attention_gqa_amd import decode, synth
    fv = decode.ForkVerify(N, seed=0, device="cuda:0", block=0, preset=dict(synth.PRESETS["fork"], vocab=1024))
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for pass_id in (0, 1):
            fv.attention(pass_id, stream)
        torch.cuda.synchronize()
        for pass_id in (0, 1):
            for _ in range(reps):
                fv.attention(pass_id, stream)
    torch.cuda.synchronize()
    print(json.dumps({"fork_rollouts": N, "calls_per_pass": reps + 1,
                      "flops_per_call": [fv.attention_flops(0), fv.attention_flops(1)]}), flush=True)


def verify_pass(N=64, reps=10):
    """The fork round's verify scan at N rollouts (24 logit rows of 151936
    per rollout), greedy and then with Gumbel noise, each issued reps times
    after one warm call; then a 256 MiB device-to-device copy whose
    FETCH_SIZE / WRITE_SIZE readings calibrate the counters."""
    import torch
    from block_causal_attention_gqa_amd import decode
    stream = torch.cuda.Stream()
    out = {"fork_rollouts": N, "calls": reps + 1}
    for temperature in (None, 0.7):
        fv = decode.ForkVerify(N, seed=0, device="cuda:0", block=0, temperature=temperature)
        with torch.cuda.stream(stream):
            for _ in range(reps + 1):
                fv.verify(stream)
        torch.cuda.synchronize()
        out["logit_bytes" if temperature is None else "logit_and_noise_bytes"] = \
            N * fv.R * fv.V * 4 * (1 if temperature is None else 2)
        del fv
        torch.cuda.empty_cache()
    src = torch.ones(64 << 20, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    out["copy_bytes"] = src.numel() * 4
    print(json.dumps(out), flush=True)


def batch_pass(S=16, L=2176, n_caches=5, reps=10):
    """The large-block decode's attention call at batch 16 (32q/8kv heads,
    head_dim 128, one 32-row block over a 2176-key prefix per sequence),
    issued reps times in rotation over n_caches distinct seeded caches (so
    no call finds its K/V in the MALL), after one warm call; then a 256 MiB
    device-to-device copy whose FETCH_SIZE / WRITE_SIZE readings calibrate
    the counters."""
    import torch
    from block_causal_attention_gqa_amd import binding as B
    from block_causal_attention_gqa_amd import synth
    dev = "cuda:0"
    R, Hq, Hkv, D = 32, 32, 8, 128
    caches = []
    for i in range(n_caches):
        (pk, pv), _ = synth.kv_cache(i, S, Hkv, L, D, [L] * S, "bf16")
        caches.append(B.KVCache(pk.to(dev), pv.to(dev)))
    (q, _), (k, _), (v, _) = synth.active_qkv(0, S, R, Hq, Hkv, D, "bf16", 0)
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty((S, R, Hq, D), dtype=torch.bfloat16, device=dev)
    ws = torch.zeros(B.bc_attn_workspace_bytes(caches[0], None, (S, R, Hq, D), [0, R]), dtype=torch.uint8, device=dev)
    for i in range(reps + 1):
        B.bc_attn_step(caches[i % n_caches], [L] * S, None, None, q, k, v, [0, R], B.BC_MASK_BLOCK_BIDIR, D ** -0.5,
                       o, ws)
    torch.cuda.synchronize()
    src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    nbytes = attn_bytes_flops(L, R, Hq, Hkv, D)[0] * S
    print(json.dumps({"calls": reps + 1, "bytes_per_call": nbytes, "copy_bytes": src.numel() * 4}), flush=True)


def pmc_pass(dec):
    """One decode's attention-partial launches (the kernel the roofline
    covers), then a plain 256 MiB device-to-device copy whose FETCH_SIZE /
    WRITE_SIZE readings calibrate the counters (expected 256 MiB each)."""
    import torch
    from block_causal_attention_gqa_amd import binding as B
    dec.run()                # warm; the cache ends committed to full length
    torch.cuda.synchronize()
    length = dec.len0.copy()
    n = 0
    for b, bs in enumerate(dec.blocks):
        for st in range(dec.steps):
            q, k, v = dec.qkv[b][st]
            B.bc_attn_partial(dec.cache, length.copy(), None, None, q, k, v, [0, bs], B.BC_MASK_BLOCK_BIDIR,
                              dec.scale, dec.out[bs], dec.ws_attn)
            n += 1
        length += bs          # the warm run already wrote the block's K/V
    torch.cuda.synchronize()
    src = torch.ones(64 << 20, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"partial_launches": n, "copy_bytes": src.numel() * 4}), flush=True)


def graph_us(fn, stream, reps=10, replays=5):
    """Average duration of one fn() on `stream`: reps calls captured back to
    back in a graph, replayed between two events on that stream."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        fn()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(reps):
                fn()
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(replays):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (replays * reps)


def make_flush(device="cuda:0"):
    """A 512 MiB buffer that evicts the 256 MB MALL and the L2s, and the
    two ways of passing it: ("dirty") writing all of it, which leaves every
    cache full of dirty lines whose write-back the next call pays for; and
    ("clean") reading one float of every 128-byte line (an elementwise
    kernel into a 16 MiB output), which leaves them full of clean lines."""
    import torch
    buf = torch.empty(128 << 20, dtype=torch.float32, device=device)
    buf.fill_(1.0)
    lines = buf.view(-1, 32)[:, 0]
    small = torch.empty(lines.numel(), dtype=torch.float32, device=device)
    return {"dirty": lambda: buf.fill_(1.0), "clean": lambda: torch.neg(lines, out=small), "bytes": buf.numel() * 4}


def cold_warm_us(stream, fn, flush, reps=20, replays=5):
    """(cold dirty, cold clean, warm) duration of one fn() on `stream`: one
    graph holds reps repetitions of [pre, fn()], another the same pre alone,
    and the call time is their difference / reps.  Cold: pre is one of the
    flushes of make_flush(), after which the MALL and the L2 hold none of the
    call's data; warm: pre is a GPU spin that touches no memory (the call's
    data stay where the previous call left them).  Median over the replays."""
    import torch

    def graph_ms(body):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            body()
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=stream):
                body()
            ts = []
            for _ in range(replays):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                g.replay()
                e1.record(stream)
                ts.append((e0, e1))
        torch.cuda.synchronize()
        return float(np.median([e0.elapsed_time(e1) for e0, e1 in ts]))

    res = []
    for state in ("dirty", "clean", "warm"):
        def pre():
            if state == "warm":
                torch.cuda._sleep(100000)
            else:
                flush[state]()

        def with_call():
            for _ in range(reps):
                pre()
                fn()

        def without():
            for _ in range(reps):
                pre()
        res.append((graph_ms(with_call) - graph_ms(without)) * 1e3 / reps)
    return res


def trajectory_legs(stream):
    """The shared-prefix fork decoding the whole 70-token trajectory section
    (blocks 24/23/23, 3282 shared keys, vocab 151936) with scaffold
    speculative rounds, at N = 1, 4, 16, 64 rollouts and draft agreement 0.5,
    0.8, 1.0.  Rounds are data dependent (the host reads each round's accept
    lengths), so a decode is timed whole on the wall clock with its inputs
    resident: median of 3 after one warm decode."""
    import torch
    from block_causal_attention_gqa_amd import decode
    rows = []
    for N in (1, 4, 16, 64):
        tr = decode.ForkTrajectory(N, 1.0, seed=0, device="cuda:0")
        for p in (0.5, 0.8, 1.0):
            tr.p_agree = p
            tr.run(stream)
            torch.cuda.synchronize()
            ts = []
            for _ in range(3):
                t0 = time.perf_counter()
                tr.run(stream)
                torch.cuda.synchronize()
                ts.append(time.perf_counter() - t0)
            ms = float(np.median(ts)) * 1e3
            n_rounds = sum(tr.rounds)
            rows.append({"N": N, "p_agree": p, "rounds": list(tr.rounds), "ms": round(ms, 3),
                         "round_us": round(ms * 1e3 / n_rounds, 1), "tokens": N * tr.cap,
                         "tok_s": round(N * tr.cap / ms * 1e3, 1)})
        del tr
        torch.cuda.empty_cache()
    return rows


def large_block_legs(stream):
    """The WAM-Diff2-shaped large-block decode (32q/8kv heads, head_dim 128,
    2048-token prefix, 256 output tokens, vocab 151936) at block sizes
    B = 1, 4, 8, 16, 32 (min(16, B) steps per block), batch 1 and 16 with
    independent prefixes, each decode replayed whole as one graph (four
    distinct logits / Q-K-V sets cycled over its steps); and the attention
    call of the middle block's first step timed back to back, cold and warm."""
    import torch
    from block_causal_attention_gqa_amd import binding as B
    from block_causal_attention_gqa_amd import decode, synth
    flush = make_flush()
    rows = []
    for S in (1, 16):
        for Bsz in synth.LARGE_BLOCK_SIZES:
            p = synth.large_block_preset(Bsz, n_seq=S)
            dec = decode.SectionDecode(p, seed=0, n_seq=S, device="cuda:0", logits_pool=4, qkv_pool=4)
            us = graph_us(lambda: dec.run(stream), stream, reps=1, replays=3)
            rec = {"B": Bsz, "batch": S, "denoise_steps": dec.denoise_steps, "decode_ms": round(us / 1e3, 3),
                   "step_us": round(us / dec.denoise_steps, 2), "tok_s": round(S * 256 / us * 1e6, 1)}
            b = len(dec.blocks) // 2
            L = p["prefix"] + b * Bsz
            q, k, v = dec.qkv[b][0]
            lens = [L] * S

            def call():
                B.bc_attn_step(dec.cache, lens, None, None, q, k, v, [0, Bsz], B.BC_MASK_BLOCK_BIDIR, dec.scale,
                               dec.out[Bsz], dec.ws_attn, stream=stream)
            b2b = graph_us(call, stream)
            dirty, clean, warm = cold_warm_us(stream, call, flush)
            nbytes, flops = (S * x for x in attn_bytes_flops(L, Bsz, dec.Hq, dec.Hkv, dec.D))
            rec["attn"] = {"prefix": L, "bytes": nbytes, "us_back_to_back": round(b2b, 3),
                           "us_cold_clean": round(clean, 3), "us_cold_dirty": round(dirty, 3),
                           "us_warm": round(warm, 3),
                           "TB_s_back_to_back": round(nbytes / b2b / 1e6, 3),
                           "TB_s_cold_clean": round(nbytes / clean / 1e6, 3),
                           "TB_s_cold_dirty": round(nbytes / dirty / 1e6, 3),
                           "TB_s_warm": round(nbytes / warm / 1e6, 3),
                           "hbm_frac_cold_clean": round(nbytes / clean / 1e3 / HBM_PEAK_GBS, 4),
                           "TFLOP_s_back_to_back": round(flops / b2b / 1e6, 1)}
            rows.append(rec)
            del dec
            torch.cuda.empty_cache()
    return rows


def tiny_leg(stream):
    """The tiny configuration: one denoise step of 8 rows over a 256-token
    prefix (4q/1kv heads, head_dim 64, float32), the unmask over [8 x 1024]
    logits, and the commit, replayed as one graph."""
    from block_causal_attention_gqa_amd import decode, synth
    dec = decode.SectionDecode(synth.PRESETS["tiny"], seed=0, device="cuda:0")
    us = graph_us(lambda: dec.run(stream), stream)
    return {"step_us": round(us, 3), "tokens": dec.tokens_per_decode}


def window_leg(stream):
    """One pipelined step with three active 7-token blocks (21 rows: the
    oldest fully active, the others semi-active; seeded completion ratios)
    over a 512-token prefix, 16q/2kv heads, head_dim 128, bf16, logits
    [21 x 2048]: the attention call and the unmask (with the masks restored
    before it, a 21-byte copy), each timed back to back."""
    import torch
    from block_causal_attention_gqa_amd import binding as B
    from block_causal_attention_gqa_amd import synth
    p = synth.PRESETS["pipelined"]
    Hq, Hkv, D, L = p["n_q_heads"], p["n_kv_heads"], p["head_dim"], p["prefix"]
    (pk, pv), _ = synth.kv_cache(0, 1, Hkv, L, D, [L], "bf16")
    (q, _), (k, _), (v, _) = synth.active_qkv(0, 1, 21, Hq, Hkv, D, "bf16", 0)
    cache = B.KVCache(pk.to("cuda:0"), pv.to("cuda:0"))
    q, k, v = q.to("cuda:0"), k.to("cuda:0"), v.to("cuda:0")
    off = [0, 7, 14, 21]
    out = torch.empty((1, 21, Hq, D), dtype=torch.bfloat16, device="cuda:0")
    ws = torch.zeros(B.bc_attn_workspace_bytes(cache, None, (1, 21, Hq, D), off), dtype=torch.uint8,
                     device="cuda:0")
    g = synth.rng(0, "ratio", 0)
    m0 = np.ones(21, np.uint8)
    for blk in range(3):
        m0[7 * blk + g.choice(7, size=int(g.random() * 7), replace=False)] = 0
    masked0 = torch.from_numpy(m0).to("cuda:0")
    masked = masked0.clone()
    tokens = torch.full((21,), -1, dtype=torch.int32, device="cuda:0")
    lg = torch.from_numpy(synth.logits(0, 21, p["vocab"], p["sigma"], 0)).to("cuda:0")
    nc = torch.zeros(3, dtype=torch.int32, device="cuda:0")
    wsu = torch.zeros(B.bc_unmask_workspace_bytes(21, p["vocab"]), dtype=torch.uint8, device="cuda:0")
    a_us = graph_us(lambda: B.bc_attn_step(cache, [L], None, None, q, k, v, off, B.BC_MASK_BLOCK_BIDIR, D ** -0.5,
                                           out, ws, stream=stream), stream)

    def unmask():
        masked.copy_(masked0)
        B.bc_unmask_select(lg, off, [B.BC_UNMASK_FULL, B.BC_UNMASK_SEMI, B.BC_UNMASK_SEMI], [1 << 30, 1, 1],
                           p["threshold"], masked, tokens, None, nc, wsu, stream=stream)
    u_us = graph_us(unmask, stream)
    nbytes = 2 * Hkv * (L + 21) * D * 2 + 2 * 21 * Hq * D * 2
    return {"attn_us": round(a_us, 3), "unmask_us_with_mask_copy": round(u_us, 3),
            "step_us": round(a_us + u_us, 3), "attn_bytes": nbytes, "attn_TB_s": round(nbytes / a_us / 1e6, 4),
            "masked_rows": int(m0.sum())}


def legs(stream):
    """Secondary measurements on the other workloads of the pages' systems:
    the shared-prefix fork round at N = 4, 16, 64 rollouts (attention there
    is MFMA-bound) with the verify scan over N = 64 rollouts' logits
    (HBM-bound); the whole fork trajectory with speculative rounds per N and
    draft agreement; the large-block decode per block size and batch with its
    attention cold and warm; the tiny float32 step; one three-block pipelined
    step; the section decode with scaffold rows inside its blocks under block
    and section visibility; a pipelined-parallel decode of 625 tokens against
    the same decode without overlap; and the duration of a minimal kernel as
    the launch floor."""
    import torch
    from block_causal_attention_gqa_amd import binding as B
    from block_causal_attention_gqa_amd import decode, synth
    out = {}
    fork = []
    for N in (4, 16, 64):
        fv = decode.ForkVerify(N, seed=0, device="cuda:0", block=0)
        rec = {"N": N, "rows": N * fv.R, "shared_prefix": fv.prefix}
        for pass_id, name in ((0, "draft_bidir"), (1, "verify_causal")):
            us = graph_us(lambda: fv.attention(pass_id, stream), stream)
            fl = fv.attention_flops(pass_id)
            rec[name] = {"attn_us": round(us, 3), "TFLOP_s": round(fl / us / 1e6, 1),
                         "mfma_frac": round(fl / us / 1e6 / BF16_PEAK_TFLOPS, 4)}
        rec["draft_argmax_us"] = round(graph_us(lambda: fv.draft_argmax(stream), stream), 3)
        vus = graph_us(lambda: fv.verify(stream), stream)
        vbytes = N * fv.R * fv.V * 4
        rec["verify"] = {"us": round(vus, 3), "GB_s": round(vbytes / vus / 1e3, 1),
                         "hbm_frac": round(vbytes / vus / 1e3 / HBM_PEAK_GBS, 4)}
        rec["round_us"] = round(graph_us(lambda: fv.run(stream), stream, reps=4), 3)
        if N == 64:
            # trajectory-only sampling: the verify also reads the Gumbel noise
            fs = decode.ForkVerify(N, seed=0, device="cuda:0", block=0, temperature=0.7)
            sus = graph_us(lambda: fs.verify(stream), stream)
            rec["verify_sampled"] = {"us": round(sus, 3), "GB_s": round(2 * vbytes / sus / 1e3, 1),
                                     "hbm_frac": round(2 * vbytes / sus / 1e3 / HBM_PEAK_GBS, 4)}
            del fs
        fork.append(rec)
        del fv
        torch.cuda.empty_cache()
    out["fork_round"] = fork

    out["trajectory"] = trajectory_legs(stream)
    out["large_block"] = large_block_legs(stream)
    out["tiny_step"] = tiny_leg(stream)
    out["pipelined_3x7"] = window_leg(stream)
    # the section decode with the sections' scaffold rows inside the blocks
    # (404 rows, 280 editable), block and section visibility, each decode
    # replayed whole as one graph like the headline
    scf = {}
    for vis in ("block", "section"):
        dec = decode.SectionDecode(synth.PRESETS["section_scaffold"], seed=0, device="cuda:0", visibility=vis)
        us = graph_us(lambda: dec.run(stream), stream, reps=1, replays=5)
        scf[vis] = {"decode_ms": round(us / 1e3, 3), "tok_s": round(dec.tokens_per_decode / us * 1e6, 1),
                    "rows": sum(dec.blocks), "units": len(dec.units), "max_unit_rows": max(dec.unit_rows)}
        del dec
        torch.cuda.empty_cache()
    out["section_scaffold"] = scf
    # pipelined parallel decoding of a 625-token output (blocks of 32 and a
    # last of 17 over a 512-token prefix, 16q/2kv heads, vocab 2048): each
    # step's commit counts decide the next step's blocks, so the host reads
    # them back every step and a decode is timed whole on the wall clock,
    # inputs resident; "sequential" is the same decode without overlap.
    # Three drivers: the schedule on the device (bc_pipeline_dev_*: every
    # step is the model stand-in's copy of its seeded outputs, the attention,
    # the unmask and the schedule kernel, replayed as graphs of 8 steps; the
    # headline figures), the library's host-side step loop
    # (bc_pipeline_decode, the counts polled in mapped host memory:
    # "native_loop"), and the step loop in Python over prepared calls
    # ("host_loop", run first: its trace bounds the staged model outputs)
    pip = {}
    for name, kw in (("pipelined", dict(add=0.5, act=0.9)), ("sequential", dict(add=1.0, act=1.0))):
        pd = decode.PipelinedDecode(seed=0, device="cuda:0", tau=0.5, n_div=4, window=3, **kw)
        pd.keep_inputs = True
        res = {}
        for driver, fn in (("host_loop", pd.run), ("native_loop", pd.run_native), ("device", pd.run_device)):
            fn(stream)
            torch.cuda.synchronize()
            reps = 5
            t0 = time.perf_counter()
            for _ in range(reps):
                n = fn(stream)
            torch.cuda.synchronize()
            ms = (time.perf_counter() - t0) * 1e3 / reps
            res[driver] = {"steps": n, "ms": round(ms, 3), "step_us": round(ms * 1e3 / n, 2),
                           "tok_s": round(sum(pd.blocks) / ms * 1e3, 1)}
        pip[name] = dict(res["device"], max_active=max(len(st["active"]) for st in pd.trace),
                         native_loop=res["native_loop"], host_loop=res["host_loop"])
        del pd
    out["pipelined_625"] = pip
    # latency floors: a one-element fill kernel, and an in-place add of 256
    # floats (two loads and one store per lane).  An add, not a copy: a
    # device-to-device copy is captured as a memcpy node, not a kernel.
    x = torch.zeros(1, device="cuda:0")
    out["launch_floor_us"] = round(graph_us(lambda: x.fill_(1.0), stream, reps=50), 3)
    src, dst = torch.ones(256, device="cuda:0"), torch.zeros(256, device="cuda:0")
    out["load_floor_us"] = round(graph_us(lambda: dst.add_(src), stream, reps=50), 3)
    return out


def cpu_baseline(dec, args, timed_out):
    """The float64 oracle on the host cores: the whole section decode (same
    seeded inputs, 88 denoise steps: attention + unmask each, commit per
    block), repeated until about --cpu-seconds have passed, in decoded tokens
    per second."""
    import threadpoolctl
    from oracle import section as OS
    from block_causal_attention_gqa_amd import synth

    seed = args.seed
    (_, _), (k32, v32) = synth.kv_cache(seed, 1, dec.Hkv, dec.cap, dec.D, [dec.prefix], dec.dtype)
    # inputs first (not timed): the same seeded tensors the GPU decode uses
    inputs = {}
    for b, bs in enumerate(dec.blocks):
        for st in range(dec.steps):
            (_, q), (_, k), (_, v) = synth.active_qkv(seed, 1, bs, dec.Hq, dec.Hkv, dec.D, dec.dtype, b, st)
            inputs[(b, st)] = (q, k, v, synth.logits(seed, bs, dec.V, dec.sigma, b, st))
    n = sum(dec.blocks)
    units = [[b] for b in range(len(dec.blocks))]
    # One untimed run with the decision trace: the decoded tokens against the
    # GPU decode's, and how close the float64 confidences came to each
    # decision (the GPU scans in float32 and re-takes, in float64, every
    # decision within a relative 2^-12 of its threshold or rank cut).
    trace = []
    ref = OS.section_decode(k32[0], v32[0], dec.prefix, units, dec.blocks, lambda b, st: inputs[(b, st)],
                            dec.steps, dec.tau, np.ones(n, np.uint8), np.full(n, -1, np.int32), scale=dec.scale,
                            attend_all=False, trace=trace)
    check = oracle_check(ref, trace, dec, timed_out)
    tokens, reps = 0, 0
    t0 = time.perf_counter()
    while True:
        OS.section_decode(k32[0], v32[0], dec.prefix, units, dec.blocks, lambda b, st: inputs[(b, st)], dec.steps,
                          dec.tau, np.ones(n, np.uint8), np.full(n, -1, np.int32), scale=dec.scale)
        tokens += n
        reps += 1
        if time.perf_counter() - t0 >= args.cpu_seconds or reps >= 50:
            break
    secs = time.perf_counter() - t0
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    return {"value": round(tokens / secs, 3), "unit": "tok/s", "cores": threads, "kind": "oracle",
            "sample": "%d repetitions of the whole section decode (%d tokens, %d denoise steps each) on "
                      "the same inputs; BLAS threads %d, os.cpu_count()=%s"
                      % (reps, n, dec.denoise_steps, threads, os.cpu_count()),
            "seconds": round(secs, 2)}, check


def oracle_check(ref, trace, dec, timed_out):
    """The oracle decode against the output of the last timed graph replay
    (tokens, masks and the committed cache), and the smallest relative
    float64 margins of its decisions: |conf - tau| / conf over the masked
    rows of every step, and (c_(k-1) - c_k) / c_(k-1) at every rank cut
    (steps whose commit count is neither 0, all masked rows nor exactly the
    rows above tau)."""
    band = 2.0 ** -12
    tau = float(np.float32(dec.tau))
    thr, cut, n_cuts, inside = float("inf"), float("inf"), 0, 0
    for _, _, conf, k in trace:
        c = conf[~np.isnan(conf)]
        if c.size == 0:
            continue
        m = float(np.min(np.abs(c - tau) / c))
        thr = min(thr, m)
        inside += m <= band
        n_above = int(np.sum(c > tau))
        if k not in (0, c.size, n_above):
            srt = np.sort(c)[::-1]
            g = float((srt[k - 1] - srt[k]) / srt[k - 1])
            cut = min(cut, g)
            n_cuts += 1
            inside += g <= band
    return {"compared": "last timed graph replay",
            "tokens_match": bool(np.array_equal(timed_out["tokens"], ref["tokens"])),
            "masked_match": bool(np.array_equal(timed_out["masked"], ref["masked"])),
            "cache_match": bool(np.array_equal(timed_out["cache_k"], ref["cache_k"])
                                and np.array_equal(timed_out["cache_v"], ref["cache_v"])),
            "steps": len(trace), "rank_cuts": n_cuts,
            "min_threshold_margin_rel": thr, "min_rank_cut_gap_rel": cut if n_cuts else None,
            "band_rel": band, "decisions_inside_band": inside}


if __name__ == "__main__":
    main()
