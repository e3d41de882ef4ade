"""Pipelined parallel decoding on the GPU (Fast-dVLA notes, key design 4):
the scheduler that drives the attention, unmask and commit calls is checked
against the float64 schedule oracle on the same seeded model outputs -- every
step's active blocks, modes and commit counts, the decoded tokens, sampled
steps' attention outputs, and the cache the in-order commits leave."""

import numpy as np
import pytest

from oracle import attention as OA, pipeline as OP
from tests import gpu_util as G
from block_causal_attention_gqa_amd import synth

pytestmark = pytest.mark.gpu

SEED = 9
P = synth.PRESETS["pipelined_625"]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    G.require_lib()


def _logits_for(b, s):
    x = synth.logits(SEED, P["blocks"][b], P["vocab"], P["sigma"], 700 + b, s)
    synth.plant_peaks(x, SEED, 0.2, 12.0, 700 + b, s)
    return x


def _qkv32(b, s):
    (_, q), (_, k), (_, v) = synth.active_qkv(SEED, 1, P["blocks"][b], P["n_q_heads"], P["n_kv_heads"],
                                              P["head_dim"], P["dtype"], 800 + b, s)
    return q, k, v


SETTINGS = [
    (0.5, 0.9, 0.5, 4, 3),     # three blocks in flight, semi phase
    (0.25, 0.5, 0.5, 8, 3),    # early joins, slow full blocks
    (1.0, 1.0, 0.5, 4, 3),     # no overlap: plain block-by-block decoding
    (0.0, 0.0, 0.9, 2, 2),     # successor full once its predecessor reveals a row, window 2
]


def _oracle(add, act, tau, n_div, window):
    return OP.pipelined_decode(list(P["blocks"]), _logits_for, add, act, tau, n_div, window)


def _sample_steps(want_trace):
    n_steps = len(want_trace)
    widest = max(range(n_steps), key=lambda k: len(want_trace[k]["active"]))
    return sorted({0, widest, n_steps // 2, n_steps - 1})


def _check(pd, want_tok, want_trace, seen):
    """Trace, tokens, sampled steps' attention and the final cache against
    the oracle's decode."""
    sizes = list(P["blocks"])
    assert len(pd.trace) == len(want_trace)
    for k, (got, want) in enumerate(zip(pd.trace, want_trace)):
        assert got == want, "step %d: %s != %s" % (k, got, want)
    assert np.array_equal(pd.tokens.cpu().numpy(), np.concatenate(want_tok))
    assert not pd.masked.cpu().numpy().any()

    # the step at which each block was last active: its K/V are the ones committed
    last = {}
    for k, st in enumerate(want_trace):
        for b in st["active"]:
            last[b] = sum(1 for x in want_trace[:k + 1] if b in x["active"]) - 1
    (_, _), (pk, pv) = synth.kv_cache(SEED, 1, P["n_kv_heads"], pd.cap, P["head_dim"], [P["prefix"]], P["dtype"])
    D = P["head_dim"]
    assert seen
    for k, (active, steps, length, got) in seen.items():
        done = [b for st in want_trace[:k] for b in st["committed"]]
        assert length == P["prefix"] + sum(sizes[b] for b in done)
        ck = np.concatenate([pk[0, :, :P["prefix"]]] + [_qkv32(b, last[b])[1][0] for b in done], axis=1)
        cv = np.concatenate([pv[0, :, :P["prefix"]]] + [_qkv32(b, last[b])[2][0] for b in done], axis=1)
        h = [_qkv32(b, s) for b, s in zip(active, steps)]
        assert [want_trace[k]["active"], [sum(1 for x in want_trace[:k] if b in x["active"]) for b in active]] == \
            [active, steps]
        q = np.concatenate([x[0] for x in h], axis=1)
        ka = np.concatenate([x[1] for x in h], axis=2)
        va = np.concatenate([x[2] for x in h], axis=2)
        off = np.concatenate([[0], np.cumsum([sizes[b] for b in active])])
        want = OA.attention_step(q, ck[None], cv[None], [length], ka, va, off, OA.MASK_BIDIR, scale=D ** -0.5)
        err = np.abs(got[:, :off[-1]] - want).max()
        assert err <= 1e-2, "step %d attention max-abs %.3g" % (k, err)

    # the cache holds the prefix, then every block's last-step K/V, in block order
    kc = pd.cache.k.float().cpu().numpy()[0]
    vc = pd.cache.v.float().cpu().numpy()[0]
    assert int(pd.length[0]) == pd.cap
    row = P["prefix"]
    for b, n in enumerate(sizes):
        _, kb, vb = _qkv32(b, last[b])
        assert np.array_equal(kc[:, row:row + n], kb[0]) and np.array_equal(vc[:, row:row + n], vb[0]), b
        row += n
    assert np.array_equal(kc[:, :P["prefix"]], pk[0, :, :P["prefix"]])


@pytest.mark.parametrize("native", [False, True], ids=["host-loop", "native-loop"])
@pytest.mark.parametrize("add,act,tau,n_div,window", SETTINGS)
def test_pipelined_625_matches_oracle(add, act, tau, n_div, window, native):
    """Both host-side drivers: the step loop in Python over prepared calls,
    and the library's own loop (bc_pipeline_decode)."""
    import torch
    from block_causal_attention_gqa_amd import decode
    print("pipelined 625 add=%g act=%g tau=%g n=%d window=%d native=%d" % (add, act, tau, n_div, window, native),
          flush=True)
    want_tok, want_trace = _oracle(add, act, tau, n_div, window)
    sample = _sample_steps(want_trace)
    pd = decode.PipelinedDecode(seed=SEED, device=G.DEV, add=add, act=act, tau=tau, n_div=n_div, window=window)
    seen = {}

    def after_attn(k, active, steps, length, out):
        if k in sample:
            torch.cuda.synchronize()
            seen[k] = (active, steps, length, out.float().cpu().numpy())

    assert (pd.run_native if native else pd.run)(after_attn=after_attn) == len(want_trace)
    torch.cuda.synchronize()
    _check(pd, want_tok, want_trace, seen)


@pytest.mark.parametrize("add,act,tau,n_div,window", SETTINGS)
def test_device_schedule_matches_oracle(add, act, tau, n_div, window):
    """The schedule on the device (bc_pipeline_dev_*): the decode replayed
    as graphs of 16 steps until the schedule kernel reports the end, then
    again step by step with every sampled step's attention read back; both
    against the oracle."""
    import torch
    from block_causal_attention_gqa_amd import decode
    print("pipelined 625 device schedule add=%g act=%g tau=%g n=%d window=%d" % (add, act, tau, n_div, window),
          flush=True)
    want_tok, want_trace = _oracle(add, act, tau, n_div, window)
    max_local = 1 + max(sum(1 for st in want_trace if b in st["active"]) for b in range(len(P["blocks"])))
    pd = decode.PipelinedDecode(seed=SEED, device=G.DEV, add=add, act=act, tau=tau, n_div=n_div, window=window)
    for rep in range(2):   # the second replays the captured graph from a reset state
        assert pd.run_device(max_local=max_local) == len(want_trace)
        torch.cuda.synchronize()
        assert pd.trace == want_trace, "graph replay %d: trace" % rep
        assert np.array_equal(pd.tokens.cpu().numpy(), np.concatenate(want_tok))
    sample = _sample_steps(want_trace)
    seen = {}

    def after_step(k, active, steps, length, out):
        if k in sample:
            seen[k] = (active, steps, length, out.float().cpu().numpy())

    # step by step, over a fresh copy of the prefix (the graph runs appended to the cache)
    (pk, pv), _ = synth.kv_cache(SEED, 1, P["n_kv_heads"], pd.cap, P["head_dim"], [P["prefix"]], P["dtype"])
    pd.cache.k.copy_(pk.to(G.DEV))
    pd.cache.v.copy_(pv.to(G.DEV))
    assert pd.run_device(max_local=max_local, after_step=after_step) == len(want_trace)
    torch.cuda.synchronize()
    _check(pd, want_tok, want_trace, seen)


def test_device_schedule_stops_at_a_missing_input():
    """Model outputs staged for too few local steps: the replay marks the
    decode stopped (error 3) instead of reading past its table, and the run
    raises."""
    import torch
    from block_causal_attention_gqa_amd import decode
    print("pipelined 625 device schedule: staged inputs too short", flush=True)
    pd = decode.PipelinedDecode(seed=SEED, device=G.DEV)
    with pytest.raises(RuntimeError, match="error 3"):
        pd.run_device(max_local=1)
    torch.cuda.synchronize()


def test_native_loop_stops_on_a_callback_error_and_runs_again():
    """An exception raised while providing a step's inputs stops the native
    loop (BC_ERR_CALLBACK inside, the exception itself outside); the device's
    count buffer is released, so a second decode runs to the oracle's end."""
    import torch
    from block_causal_attention_gqa_amd import decode
    print("pipelined 625 native loop: callback error, then a full decode", flush=True)
    pd = decode.PipelinedDecode(seed=SEED, device=G.DEV)
    real = pd._native_inputs
    calls = []

    def failing(active, steps):
        calls.append(1)
        if len(calls) == 4:
            raise KeyError("no inputs for this step")
        return real(active, steps)

    pd._native_inputs = failing
    with pytest.raises(KeyError):
        pd.run_native()
    torch.cuda.synchronize()
    assert len(calls) == 4
    pd._native_inputs = real
    sizes = list(P["blocks"])
    want_tok, want_trace = OP.pipelined_decode(sizes, _logits_for, pd.add, pd.act, pd.tau, pd.n_div, pd.window)
    assert pd.run_native() == len(want_trace)
    torch.cuda.synchronize()
    assert pd.trace == want_trace
    assert np.array_equal(pd.tokens.cpu().numpy(), np.concatenate(want_tok))


@pytest.mark.parametrize("add,act,n_div,window", [(0.3, 0.6, 2, 3), (0.0, 0.5, 3, 2)])
def test_irregular_blocks_all_drivers(add, act, n_div, window):
    """Blocks of 7, 1, 9, 4, 2 and 13 rows over a 100-key prefix (vocabulary
    1024): the widest step is not a multiple of any block size and a one-row
    block joins and commits; every driver against the oracle's trace and
    tokens, and the cache holding each block's K/V of its last step."""
    import torch
    from block_causal_attention_gqa_amd import decode
    print("pipelined irregular blocks add=%g act=%g n=%d window=%d" % (add, act, n_div, window), flush=True)
    preset = dict(P, blocks=[7, 1, 9, 4, 2, 13], prefix=100, vocab=1024)
    sizes = preset["blocks"]
    pd = decode.PipelinedDecode(preset, seed=SEED, device=G.DEV, add=add, act=act, tau=0.5, n_div=n_div,
                                window=window)
    want_tok, want_trace = OP.pipelined_decode(sizes, pd.logits_for, add, act, 0.5, n_div, window)
    last = {}
    for k, st in enumerate(want_trace):
        for b in st["active"]:
            last[b] = sum(1 for x in want_trace[:k + 1] if b in x["active"]) - 1
    max_local = 1 + max(last.values())
    runs = (("host", lambda: pd.run()), ("native", lambda: pd.run_native()),
            ("device", lambda: pd.run_device(max_local=max_local)))
    for name, fn in runs:
        assert fn() == len(want_trace), name
        torch.cuda.synchronize()
        assert pd.trace == want_trace, name
        assert np.array_equal(pd.tokens.cpu().numpy(), np.concatenate(want_tok)), name
        assert not pd.masked.cpu().numpy().any(), name
        kc = pd.cache.k.float().cpu().numpy()[0]
        vc = pd.cache.v.float().cpu().numpy()[0]
        assert int(pd.length[0]) == preset["prefix"] + sum(sizes), name
        row = preset["prefix"]
        for b, n in enumerate(sizes):
            _, (_, kb), (_, vb) = pd.qkv_for(b, last[b])
            assert np.array_equal(kc[:, row:row + n], kb[0]) and np.array_equal(vc[:, row:row + n], vb[0]), (name, b)
            row += n


@pytest.mark.parametrize("dtype,head_dim", [("f32", 128), ("f32", 64), ("bf16", 64)])
def test_device_plan_cases_of_other_dtypes_and_head_dims(dtype, head_dim):
    """The device-plan cases of the float32 partial kernel and of head_dim 64
    (8q/2kv heads, blocks of 5, 12, 3 and 9 rows over a 40-key prefix,
    vocabulary 512): trace, tokens and committed cache of every driver
    against the oracle, and one sampled step's attention within the
    tolerance of its dtype (1e-5 for float32, 1e-2 for bf16)."""
    import torch
    from block_causal_attention_gqa_amd import decode
    print("pipelined %s D=%d: all drivers" % (dtype, head_dim), flush=True)
    preset = dict(P, dtype=dtype, head_dim=head_dim, n_q_heads=8, n_kv_heads=2, blocks=[5, 12, 3, 9], prefix=40,
                  vocab=512)
    sizes = preset["blocks"]
    add, act, tau, n_div, window = 0.2, 0.6, 0.5, 3, 3
    pd = decode.PipelinedDecode(preset, seed=SEED, device=G.DEV, add=add, act=act, tau=tau, n_div=n_div,
                                window=window)
    want_tok, want_trace = OP.pipelined_decode(sizes, pd.logits_for, add, act, tau, n_div, window)
    last = {}
    for k, st in enumerate(want_trace):
        for b in st["active"]:
            last[b] = sum(1 for x in want_trace[:k + 1] if b in x["active"]) - 1
    max_local = 1 + max(last.values())
    tol = 1e-5 if dtype == "f32" else 1e-2
    sample = len(want_trace) // 2
    seen = {}

    def after_step(k, active, steps, length, out):
        if k == sample:
            seen[k] = (active, steps, length, out.float().cpu().numpy())

    runs = (("host", lambda: pd.run()), ("native", lambda: pd.run_native()),
            ("device", lambda: pd.run_device(max_local=max_local)),
            ("device-steps", lambda: pd.run_device(max_local=max_local, after_step=after_step)))
    for name, fn in runs:
        assert fn() == len(want_trace), name
        torch.cuda.synchronize()
        assert pd.trace == want_trace, name
        assert np.array_equal(pd.tokens.cpu().numpy(), np.concatenate(want_tok)), name
        kc = pd.cache.k.float().cpu().numpy()[0]
        vc = pd.cache.v.float().cpu().numpy()[0]
        row = preset["prefix"]
        for b, n in enumerate(sizes):
            _, (_, kb), (_, vb) = pd.qkv_for(b, last[b])
            assert np.array_equal(kc[:, row:row + n], kb[0]) and np.array_equal(vc[:, row:row + n], vb[0]), (name, b)
            row += n
    # the sampled step against the oracle's attention over the cache it saw
    active, steps, length, got = seen[sample]
    done = [b for st in want_trace[:sample] for b in st["committed"]]
    assert length == preset["prefix"] + sum(sizes[b] for b in done)
    (_, _), (pk, pv) = synth.kv_cache(SEED, 1, preset["n_kv_heads"], pd.cap, head_dim, [preset["prefix"]], dtype)
    ck = np.concatenate([pk[0, :, :preset["prefix"]]] + [pd.qkv_for(b, last[b])[1][1][0] for b in done], axis=1)
    cv = np.concatenate([pv[0, :, :preset["prefix"]]] + [pd.qkv_for(b, last[b])[2][1][0] for b in done], axis=1)
    h = [pd.qkv_for(b, s) for b, s in zip(active, steps)]
    q = np.concatenate([x[0][1] for x in h], axis=1)
    ka = np.concatenate([x[1][1] for x in h], axis=2)
    va = np.concatenate([x[2][1] for x in h], axis=2)
    off = np.concatenate([[0], np.cumsum([sizes[b] for b in active])])
    want = OA.attention_step(q, ck[None], cv[None], [length], ka, va, off, OA.MASK_BIDIR, scale=head_dim ** -0.5)
    err = np.abs(got[:, :off[-1]] - want).max()
    assert err <= tol, "sampled step %d attention max-abs %.3g" % (sample, err)


@pytest.mark.parametrize("add,act", [(0.5, 0.9), (1.0, 1.0)])
def test_bench_configurations_all_drivers(add, act):
    """The 625-token decode exactly as the bench times it (seed 0, tau 0.5,
    n = 4, window 3; with overlap and without): every driver's trace, tokens
    and final cache length against the oracle."""
    import torch
    from block_causal_attention_gqa_amd import decode
    print("pipelined 625 bench configuration add=%g act=%g" % (add, act), flush=True)
    pd = decode.PipelinedDecode(seed=0, device=G.DEV, tau=0.5, n_div=4, window=3, add=add, act=act)
    want_tok, want_trace = OP.pipelined_decode(list(P["blocks"]), pd.logits_for, add, act, 0.5, 4, 3)
    pd.keep_inputs = True
    for name, fn in (("host", pd.run), ("native", pd.run_native), ("device", pd.run_device)):
        assert fn() == len(want_trace), name
        torch.cuda.synchronize()
        assert pd.trace == want_trace, name
        assert np.array_equal(pd.tokens.cpu().numpy(), np.concatenate(want_tok)), name
        assert int(pd.length[0]) == pd.cap, name
