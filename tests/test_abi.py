"""The C-ABI library loads, exports every entry point include/bc.h declares,
and rejects malformed arguments on the host before any launch.

Every call here fails host-side validation by construction, so no kernel is
launched and no pointer is dereferenced: the tests run without a GPU."""

import ctypes
import os
import re

import pytest

from block_causal_attention_gqa_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    with open(os.path.join(ROOT, "include", "bc.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char|void|bc_\w+)\s*\*?\s*(bc_\w+)\s*\(", text,
                                 re.M)))


@pytest.fixture(scope="module")
def L():
    import torch
    if torch.cuda.is_available():
        # host-only checks; on a GPU machine the parity tests cover the library
        pytest.skip("host-side ABI checks run where no GPU is present")
    return B.lib()


def test_header_and_binding_agree():
    assert declared_functions() == sorted(B.EXPORTED)


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings(L):
    for st in range(-8, 1):
        assert B.bc_status_str(st).startswith("BC_")
    assert B.bc_status_str(-99) == "unknown bc_status"


def _cache(dtype=B.BC_BF16, S=1, Hkv=2, D=128, cap=64, k=1, v=1):
    return B.BcKvCache(k, v, dtype, S, Hkv, D, cap)


def _active(S=1, R=8, Hq=16, off=(0, 8)):
    arr = (ctypes.c_int32 * len(off))(*off)
    return B.BcActive(1, 1, 1, ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32)), len(off) - 1, S, R, Hq), arr


def _lens(*xs):
    return (ctypes.c_int32 * len(xs))(*xs)


def attn(L, cache, lens, act, mask=0, splits=0, ws=1, ws_bytes=1 << 40, priv=None, priv_len=None, out=1):
    return L.bc_attn_step(ctypes.byref(cache), lens, ctypes.byref(priv) if priv else None, priv_len,
                          ctypes.byref(act), mask, 0.1, splits, out, ws, ws_bytes, None)


def test_attention_validation(L):
    act, keep = _active()
    assert attn(L, _cache(D=96), _lens(8), act) == B.BC_ERR_UNSUPPORTED
    assert attn(L, _cache(dtype=7), _lens(8), act) == B.BC_ERR_UNSUPPORTED
    assert attn(L, _cache(k=0), _lens(8), act) == B.BC_ERR_ARG
    assert attn(L, _cache(Hkv=3), _lens(8), act) == B.BC_ERR_ARG          # 16 % 3
    assert attn(L, _cache(), _lens(65), act) == B.BC_ERR_ARG              # > capacity
    assert attn(L, _cache(), _lens(-1), act) == B.BC_ERR_ARG
    assert attn(L, _cache(), _lens(8), act, mask=2) == B.BC_ERR_ARG
    assert attn(L, _cache(), _lens(8), act, splits=257) == B.BC_ERR_ARG
    assert attn(L, _cache(), _lens(8), act, ws=0) == B.BC_ERR_WORKSPACE
    assert attn(L, _cache(), _lens(8), act, ws_bytes=16) == B.BC_ERR_WORKSPACE
    assert attn(L, _cache(), _lens(8), act, out=0) == B.BC_ERR_ARG
    assert attn(L, _cache(S=2), _lens(8, 8), act) == B.BC_ERR_ARG        # n_seq mismatch
    bad, k1 = _active(off=(0, 4, 4, 8))
    assert attn(L, _cache(), _lens(8), bad) == B.BC_ERR_ARG
    bad, k2 = _active(off=(1, 8))
    assert attn(L, _cache(), _lens(8), bad) == B.BC_ERR_ARG
    bad, k3 = _active(off=(0, 7))
    assert attn(L, _cache(), _lens(8), bad) == B.BC_ERR_ARG
    many, k4 = _active(S=B.BC_MAX_SEQ + 1)
    assert attn(L, _cache(S=B.BC_MAX_SEQ + 1), _lens(*([8] * (B.BC_MAX_SEQ + 1))), many) == B.BC_ERR_UNSUPPORTED
    blocks, k5 = _active(R=70, off=tuple(range(71)))
    assert attn(L, _cache(), _lens(8), blocks) == B.BC_ERR_UNSUPPORTED  # > BC_MAX_BLOCKS
    # fork: shared prefix must hold one sequence, priv one per rollout
    f_act, k6 = _active(S=2)
    assert attn(L, _cache(S=2), _lens(8, 8), f_act, priv=_cache(S=2), priv_len=_lens(0, 0)) == B.BC_ERR_ARG
    assert attn(L, _cache(S=1), _lens(8), f_act, priv=_cache(S=3), priv_len=_lens(0, 0)) == B.BC_ERR_ARG
    assert attn(L, _cache(S=1), _lens(8), f_act, priv=_cache(S=2), priv_len=None) == B.BC_ERR_ARG
    assert attn(L, _cache(S=1), _lens(8), f_act, priv=_cache(S=2), priv_len=_lens(0, 65)) == B.BC_ERR_ARG
    assert attn(L, _cache(S=1), _lens(8), f_act, priv=_cache(S=2, dtype=B.BC_F32),
                priv_len=_lens(0, 0)) == B.BC_ERR_UNSUPPORTED


def test_static_attention_validation(L):
    # the allocation-free entry point validates like bc_attn_step, before it
    # looks up its scratch on the device
    def call(cache, lens, act, mask=0, splits=0, out=1):
        return L.bc_attn_step_static(ctypes.byref(cache), lens, None, None, ctypes.byref(act), mask, 0.1, splits,
                                     out, None)
    act, keep = _active()
    assert call(_cache(D=96), _lens(8), act) == B.BC_ERR_UNSUPPORTED
    assert call(_cache(k=0), _lens(8), act) == B.BC_ERR_ARG
    assert call(_cache(), _lens(65), act) == B.BC_ERR_ARG
    assert call(_cache(), _lens(8), act, mask=2) == B.BC_ERR_ARG
    assert call(_cache(), _lens(8), act, splits=257) == B.BC_ERR_ARG
    assert call(_cache(), _lens(8), act, out=0) == B.BC_ERR_ARG
    assert "static scratch" in B.bc_status_str(B.BC_ERR_SCRATCH)


def test_workspace_queries(L):
    act, keep = _active()
    c = _cache(cap=3352)
    n0 = L.bc_attn_workspace_bytes(ctypes.byref(c), None, ctypes.byref(act), 0)
    n1 = L.bc_attn_workspace_bytes(ctypes.byref(c), None, ctypes.byref(act), 1)
    assert n0 > n1 > 0 and n0 % 256 == 0
    assert L.bc_attn_workspace_bytes(ctypes.byref(_cache(D=96)), None, ctypes.byref(act), 0) == 0
    chunks = -(-151936 // 4096)
    assert L.bc_unmask_workspace_bytes(32, 151936) >= 32 * chunks * 16
    assert L.bc_unmask_workspace_bytes(0, 10) == 0
    assert L.bc_verify_workspace_bytes(64, 24, 151936) >= 64 * 24 * chunks * 16


def test_commit_validation(L):
    c = _cache(cap=64)
    ln = _lens(60)
    assert L.bc_kv_commit(ctypes.byref(c), ln, 0, 59, 4, 1, 1, None) == B.BC_ERR_ORDER
    assert L.bc_kv_commit(ctypes.byref(c), ln, 0, 60, 5, 1, 1, None) == B.BC_ERR_CAPACITY
    assert L.bc_kv_commit(ctypes.byref(c), ln, 1, 60, 1, 1, 1, None) == B.BC_ERR_ARG
    assert L.bc_kv_commit(ctypes.byref(c), ln, 0, 60, 0, 1, 1, None) == B.BC_ERR_ARG
    assert L.bc_kv_commit(ctypes.byref(c), ln, 0, 60, 1, 0, 1, None) == B.BC_ERR_ARG
    assert L.bc_kv_commit(ctypes.byref(_cache(D=80)), ln, 0, 60, 1, 1, 1, None) == B.BC_ERR_UNSUPPORTED
    assert ln[0] == 60
    c2, ln2 = _cache(S=3, cap=64), _lens(10, 10, 11)
    assert L.bc_kv_commit(ctypes.byref(c2), ln2, B.BC_ALL_SEQ, 10, 4, 1, 1, None) == B.BC_ERR_ORDER
    assert L.bc_kv_commit(ctypes.byref(c2), ln2, -2, 10, 4, 1, 1, None) == B.BC_ERR_ARG
    ln3 = _lens(62, 62, 62)
    assert L.bc_kv_commit(ctypes.byref(c2), ln3, B.BC_ALL_SEQ, 62, 3, 1, 1, None) == B.BC_ERR_CAPACITY
    assert list(ln2) == [10, 10, 11] and list(ln3) == [62, 62, 62]


def test_unmask_validation(L):
    off, mode, div = _lens(0, 4), _lens(1), _lens(2)

    def call(logits=1, R=4, V=10, off=off, nb=1, mode=mode, div=div, tau=0.9, masked=1, ws=1, wsb=1 << 30):
        return L.bc_unmask_select(logits, R, V, off, nb, mode, div, tau, masked, 1, None, 1, ws, wsb, None)
    assert call(logits=0) == B.BC_ERR_ARG
    assert call(V=0) == B.BC_ERR_ARG
    assert call(off=_lens(0, 3)) == B.BC_ERR_ARG
    assert call(mode=_lens(5)) == B.BC_ERR_ARG
    assert call(div=_lens(0)) == B.BC_ERR_ARG
    assert call(tau=float("nan")) == B.BC_ERR_ARG
    assert call(masked=0) == B.BC_ERR_ARG
    assert call(ws=0) == B.BC_ERR_WORKSPACE
    assert call(wsb=15) == B.BC_ERR_WORKSPACE
    assert call(R=2000, off=_lens(0, 2000)) == B.BC_ERR_UNSUPPORTED   # block > 1024 rows
    assert call(R=5000, off=_lens(*range(0, 5001, 1000))) == B.BC_ERR_UNSUPPORTED  # > BC_MAX_SCAN_ROWS


def test_verify_validation(L):
    def call(logits=1, S=1, Lr=4, V=10, draft=1, m=4, first=1, acc=1, bonus=1, ws=1, wsb=1 << 30):
        return L.bc_spec_verify(logits, S, Lr, V, draft, m, None, first, acc, bonus, ws, wsb, None)
    assert call(m=5) == B.BC_ERR_ARG
    assert call(m=0) == B.BC_ERR_ARG
    assert call(draft=0) == B.BC_ERR_ARG
    assert call(first=0) == B.BC_ERR_ARG
    assert call(V=0) == B.BC_ERR_ARG
    assert call(ws=0) == B.BC_ERR_WORKSPACE
    assert call(wsb=100) == B.BC_ERR_WORKSPACE
    assert call(S=200, Lr=24, m=24) == B.BC_ERR_UNSUPPORTED   # 4800 rows > BC_MAX_SCAN_ROWS


def test_partial_record_sizes_follow_the_row_count(L):
    # with an explicit split count P the workspace holds (P + 1) records per
    # output row: 520 bytes (float32) below 1024 output rows or for float32
    # inputs, 272 bytes (compact int16) from 1024 rows with bf16 inputs
    def nbytes(dtype, R, Hq=16):
        act, keep = _active(R=R, Hq=Hq, off=(0, R))
        return L.bc_attn_workspace_bytes(ctypes.byref(_cache(dtype=dtype, cap=512)), None, ctypes.byref(act), 2)

    def rounded(n):
        return (n + 255) // 256 * 256
    for dtype, R, per_row in ((B.BC_BF16, 32, (512, 8)), (B.BC_BF16, 64, (256, 16)), (B.BC_F32, 64, (512, 8))):
        rows = R * 16
        assert nbytes(dtype, R) == rounded(3 * rows * per_row[0]) + rounded(3 * rows * per_row[1]), (dtype, R)


def test_fork_row_tile_form_keeps_the_split_plans_workspace(L):
    # N = 64 rollouts over a 3282-key shared prefix (24 rows x 16 heads per
    # rollout, 2 KV heads): the automatic plan is the row-tile form with one
    # key split, which writes no split partials, yet reports the split
    # plan's size (P = 2 prefix splits + the active slot, compact records),
    # so that a workspace sized for the shapes also serves calls that split
    act, keep = _active(S=64, R=24, Hq=16, off=(0, 24))
    shared, priv = _cache(S=1, cap=3282), _cache(S=64, cap=48)
    auto = L.bc_attn_workspace_bytes(ctypes.byref(shared), ctypes.byref(priv), ctypes.byref(act), 0)
    two = L.bc_attn_workspace_bytes(ctypes.byref(shared), ctypes.byref(priv), ctypes.byref(act), 2)
    rows = 64 * 24 * 16
    assert auto == two == (3 * rows * 128 * 2 + 255) // 256 * 256 + (3 * rows * 16 + 255) // 256 * 256


def test_pipeline_decode_validation(L):
    """bc_pipeline_decode checks its pointers, the one-sequence cache and the
    step bound before it touches the device."""
    h = ctypes.c_void_p()
    sizes = (ctypes.c_int32 * 2)(4, 4)
    assert L.bc_pipeline_create(sizes, 2, 2, 0.5, 0.9, 4, ctypes.byref(h)) == B.BC_OK
    lens = _lens(0)
    n = ctypes.c_int32(-5)
    fi = B.STEP_INPUTS_FN(lambda *a: 0)
    none_after = B.AFTER_ATTN_FN()

    def call(p=h, cache=None, length=lens, inputs=fi, max_steps=16, masked=1, tokens=1, out=1, n_steps=True):
        c = cache if cache is not None else _cache()
        return L.bc_pipeline_decode(p, ctypes.byref(c), length, 16, 1024, 0.1, 0.9, masked, tokens, out, 1, 1 << 20,
                                    1, 1 << 20, inputs, none_after, None, None, max_steps,
                                    ctypes.byref(n) if n_steps else None, None)

    try:
        assert call(p=None) == B.BC_ERR_ARG
        assert call(cache=_cache(S=2)) == B.BC_ERR_ARG
        assert call(length=None) == B.BC_ERR_ARG
        assert call(inputs=B.STEP_INPUTS_FN()) == B.BC_ERR_ARG
        assert call(max_steps=-1) == B.BC_ERR_ARG
        assert call(masked=None) == B.BC_ERR_ARG
        assert call(tokens=None) == B.BC_ERR_ARG
        assert call(out=None) == B.BC_ERR_ARG
        assert call(n_steps=False) == B.BC_ERR_ARG
        assert n.value == -5   # nothing written on a rejected call
    finally:
        L.bc_pipeline_destroy(h)


def test_device_pipeline_validation(L):
    """bc_pipeline_dev_create rejects malformed schedules, caches and
    buffers on the host; the other bc_pipeline_dev_* calls reject a null
    handle."""
    sizes = (ctypes.c_int32 * 3)(32, 32, 17)
    out = ctypes.c_void_p()

    def create(n_blocks=3, window=2, n_div=4, cache=None, prefix=16, masked=1, q=1, max_steps=100, vocab=1024):
        c = cache if cache is not None else _cache(cap=512)
        return L.bc_pipeline_dev_create(sizes, n_blocks, window, 0.5, 0.9, n_div, ctypes.byref(c), prefix, 16, vocab,
                                        0.1, 0.9, masked, 1, q, 1, 1, 1, 1, max_steps, ctypes.byref(out))

    assert create(n_blocks=0) == B.BC_ERR_ARG
    assert create(window=0) == B.BC_ERR_ARG
    assert create(n_div=0) == B.BC_ERR_ARG
    assert create(cache=_cache(S=2, cap=512)) == B.BC_ERR_ARG
    assert create(prefix=512 - 80) == B.BC_ERR_ARG        # the blocks would not fit
    assert create(masked=None) == B.BC_ERR_ARG
    assert create(q=None) == B.BC_ERR_ARG
    assert create(max_steps=0) == B.BC_ERR_ARG
    assert create(vocab=0) == B.BC_ERR_ARG
    assert create(vocab=1022) == B.BC_ERR_UNSUPPORTED   # logit rows not whole 16-byte units
    assert out.value is None
    for f in (L.bc_pipeline_dev_reset, L.bc_pipeline_dev_step):
        assert f(None, None) == B.BC_ERR_ARG
    assert L.bc_pipeline_dev_replay(None, 1, 1, None) == B.BC_ERR_ARG
    assert L.bc_pipeline_dev_status(None, None, None, None, None) == B.BC_ERR_ARG
    assert L.bc_pipeline_dev_trace(None, None, 0) == B.BC_ERR_ARG
    assert L.bc_pipeline_dev_read_plan(None, None) == B.BC_ERR_ARG
    assert L.bc_pipeline_dev_rows(None) == B.BC_ERR_ARG
    assert L.bc_pipeline_dev_plan(None) is None


def test_one_column_tile_splits_fit_each_xcd(L):
    # bf16 calls without a fork and with at most 8 row tiles, whose items run
    # under the XCD-aligned mapping (a row tile's P + 1 items on an XCD of its
    # own, 32 CUs): the automatic split count keeps those items on a CU each,
    # P + 1 <= 32.  Over the bs1 section
    # decode's prefixes (3072-3346 keys) that is the two-tile split count
    # ceil(L / 128), where items of one tile would need 48-53 splits.  Read
    # back from the workspace size, which holds (P + 1) float32 records of 520
    # bytes per output row (fewer than 1024 rows here), each array rounded up
    # to 256 bytes.
    def auto_p(R, cap, S=1, Hq=16, Hkv=2, per_row=520):
        act, keep = _active(S=S, R=R, Hq=Hq, off=(0, R))
        n = L.bc_attn_workspace_bytes(ctypes.byref(_cache(S=S, Hkv=Hkv, cap=cap)), None, ctypes.byref(act), 0)
        return n // (S * R * Hq * per_row) - 1
    for R in (6, 12, 32):           # 2, 4 and 8 row tiles of 64 rows: one per XCD at most
        for cap in (3072, 3276, 3346):
            assert auto_p(R, cap) == -(-cap // 128), (R, cap)
        assert auto_p(R, 1000) + 1 <= 32
    # more row tiles than XCDs keep the model's count: batch 16, 32q/8kv,
    # 32-row blocks (256 row tiles) take 2 splits; 1-row blocks (128 row
    # tiles of 4 rows) more than one
    assert auto_p(32, 2176, S=16, Hq=32, Hkv=8, per_row=272) == 2
    assert auto_p(1, 2176, S=16, Hq=32, Hkv=8) > 1
