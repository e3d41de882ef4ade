"""ctypes binding of ``libbc.so`` (declared in ``include/bc.h``).

Argument marshalling only: every function here turns torch tensors and host
lists into the pointers and sizes of the C entry point of the same name and
returns its status.  All computation happens in the HIP kernels behind those
entry points; there is no fallback path.  Device tensors are checked for
device, dtype, contiguity and minimum size before their pointers are handed
over, because the C ABI cannot see tensor extents.
"""

import ctypes
import os

import numpy as np
import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbc.so")

BC_OK = 0
BC_ERR_ARG = -1
BC_ERR_UNSUPPORTED = -2
BC_ERR_CAPACITY = -3
BC_ERR_ORDER = -4
BC_ERR_WORKSPACE = -5
BC_ERR_HIP = -6
BC_ERR_SCRATCH = -7
BC_ERR_CALLBACK = -8
BC_STATIC_SCRATCH_BYTES = 32 << 20

BC_F32 = 0
BC_BF16 = 1
BC_MASK_BLOCK_BIDIR = 0
BC_MASK_BLOCK_CAUSAL = 1
BC_UNMASK_SEMI = 0
BC_UNMASK_FULL = 1
BC_MAX_SEQ = 64
BC_MAX_BLOCKS = 64
BC_MAX_BLOCK_ROWS = 1024
BC_MAX_SCAN_ROWS = 4096
BC_ALL_SEQ = -1

EXPORTED = ("bc_kv_commit", "bc_attn_workspace_bytes", "bc_attn_step", "bc_unmask_workspace_bytes",
            "bc_unmask_select", "bc_verify_workspace_bytes", "bc_spec_verify", "bc_spec_verify_sampled",
            "bc_status_str", "bc_attn_partial", "bc_attn_combine", "bc_vocab_scan", "bc_unmask_decide",
            "bc_pipeline_create", "bc_pipeline_destroy", "bc_pipeline_next", "bc_pipeline_report",
            "bc_attn_step_static", "bc_pipeline_decode", "bc_pipeline_dev_create", "bc_pipeline_dev_destroy",
            "bc_pipeline_dev_rows", "bc_pipeline_dev_plan", "bc_pipeline_dev_reset", "bc_pipeline_dev_step",
            "bc_pipeline_dev_replay", "bc_pipeline_dev_status", "bc_pipeline_dev_trace",
            "bc_pipeline_dev_read_plan")

_c_i32p = ctypes.POINTER(ctypes.c_int32)


class BcKvCache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("n_seq", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("capacity", ctypes.c_int32)]


class BcActive(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("blk_off", _c_i32p), ("n_blk", ctypes.c_int32), ("n_seq", ctypes.c_int32),
                ("n_rows", ctypes.c_int32), ("n_q_heads", ctypes.c_int32)]


class BcStepInputs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("logits", ctypes.c_void_p), ("blk_k", ctypes.c_void_p * BC_MAX_BLOCKS),
                ("blk_v", ctypes.c_void_p * BC_MAX_BLOCKS)]


class BcDevPlan(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("rows", ctypes.c_int32), ("row0", ctypes.c_int32), ("len", ctypes.c_int32),
                ("n_blk", ctypes.c_int32), ("blk_off", ctypes.c_int32 * (BC_MAX_BLOCKS + 2)),
                ("active", ctypes.c_int32 * BC_MAX_BLOCKS), ("local_step", ctypes.c_int32 * BC_MAX_BLOCKS),
                ("mode", ctypes.c_int32 * BC_MAX_BLOCKS), ("n_div", ctypes.c_int32 * BC_MAX_BLOCKS)]


class BcStepBlock(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("logits", ctypes.c_void_p)]


# bc_step_inputs_fn and bc_after_attn_fn
STEP_INPUTS_FN = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, _c_i32p, _c_i32p,
                                  ctypes.POINTER(BcStepInputs))
AFTER_ATTN_FN = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, _c_i32p, _c_i32p,
                                 ctypes.c_int32, ctypes.c_void_p)


def pipe_trace_ints(window):
    """BC_PIPE_TRACE_INTS(window): int32 entries per step of the native trace."""
    return 2 + 4 * int(window)


class BcError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__("%s: %s" % (what, bc_status_str(status)))


_lib = None


def lib():
    """Load libbc.so once.  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libbc.so is not built (%s); run `python -m block_causal_attention_gqa_amd.build`"
                           % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    cp, ap = ctypes.POINTER(BcKvCache), ctypes.POINTER(BcActive)
    L.bc_status_str.argtypes = [ctypes.c_int]
    L.bc_status_str.restype = ctypes.c_char_p
    L.bc_kv_commit.argtypes = [cp, _c_i32p, i32, i32, i32, vp, vp, vp]
    L.bc_kv_commit.restype = ctypes.c_int
    L.bc_attn_workspace_bytes.argtypes = [cp, cp, ap, i32]
    L.bc_attn_workspace_bytes.restype = sz
    for name in ("bc_attn_step", "bc_attn_partial", "bc_attn_combine"):
        f = getattr(L, name)
        f.argtypes = [cp, _c_i32p, cp, _c_i32p, ap, i32, ctypes.c_float, i32, vp, vp, sz, vp]
        f.restype = ctypes.c_int
    L.bc_attn_step_static.argtypes = [cp, _c_i32p, cp, _c_i32p, ap, i32, ctypes.c_float, i32, vp, vp]
    L.bc_attn_step_static.restype = ctypes.c_int
    L.bc_unmask_workspace_bytes.argtypes = [i32, i32]
    L.bc_unmask_workspace_bytes.restype = sz
    for name in ("bc_unmask_select", "bc_unmask_decide"):
        f = getattr(L, name)
        f.argtypes = [vp, i32, i32, _c_i32p, i32, _c_i32p, _c_i32p, ctypes.c_float, vp, vp, vp, vp, vp, sz, vp]
        f.restype = ctypes.c_int
    L.bc_vocab_scan.argtypes = [vp, i32, i32, vp, i32, vp, sz, vp]
    L.bc_vocab_scan.restype = ctypes.c_int
    L.bc_verify_workspace_bytes.argtypes = [i32, i32, i32]
    L.bc_verify_workspace_bytes.restype = sz
    L.bc_spec_verify.argtypes = [vp, i32, i32, i32, vp, i32, vp, vp, vp, vp, vp, sz, vp]
    L.bc_spec_verify.restype = ctypes.c_int
    L.bc_spec_verify_sampled.argtypes = [vp, vp, ctypes.c_float, i32, i32, i32, vp, i32, vp, vp, vp, vp, vp, sz, vp]
    L.bc_spec_verify_sampled.restype = ctypes.c_int
    L.bc_pipeline_create.argtypes = [_c_i32p, i32, i32, ctypes.c_double, ctypes.c_double, i32,
                                     ctypes.POINTER(ctypes.c_void_p)]
    L.bc_pipeline_create.restype = ctypes.c_int
    L.bc_pipeline_destroy.argtypes = [vp]
    L.bc_pipeline_destroy.restype = None
    L.bc_pipeline_next.argtypes = [vp, _c_i32p, _c_i32p, _c_i32p, _c_i32p, _c_i32p, _c_i32p]
    L.bc_pipeline_next.restype = ctypes.c_int
    L.bc_pipeline_report.argtypes = [vp, _c_i32p, _c_i32p]
    L.bc_pipeline_report.restype = ctypes.c_int
    L.bc_pipeline_decode.argtypes = [vp, cp, _c_i32p, i32, i32, ctypes.c_float, ctypes.c_float, vp, vp, vp,
                                     vp, sz, vp, sz, STEP_INPUTS_FN, AFTER_ATTN_FN, vp, _c_i32p, i32, _c_i32p, vp]
    L.bc_pipeline_decode.restype = ctypes.c_int
    L.bc_pipeline_dev_create.argtypes = [_c_i32p, i32, i32, ctypes.c_double, ctypes.c_double, i32, cp, i32, i32, i32,
                                         ctypes.c_float, ctypes.c_float, vp, vp, vp, vp, vp, vp, vp, i32,
                                         ctypes.POINTER(ctypes.c_void_p)]
    L.bc_pipeline_dev_create.restype = ctypes.c_int
    L.bc_pipeline_dev_destroy.argtypes = [vp]
    L.bc_pipeline_dev_destroy.restype = None
    L.bc_pipeline_dev_rows.argtypes = [vp]
    L.bc_pipeline_dev_rows.restype = ctypes.c_int
    L.bc_pipeline_dev_plan.argtypes = [vp]
    L.bc_pipeline_dev_plan.restype = ctypes.c_void_p
    L.bc_pipeline_dev_reset.argtypes = [vp, vp]
    L.bc_pipeline_dev_reset.restype = ctypes.c_int
    L.bc_pipeline_dev_step.argtypes = [vp, vp]
    L.bc_pipeline_dev_step.restype = ctypes.c_int
    L.bc_pipeline_dev_replay.argtypes = [vp, vp, i32, vp]
    L.bc_pipeline_dev_replay.restype = ctypes.c_int
    L.bc_pipeline_dev_status.argtypes = [vp, _c_i32p, _c_i32p, _c_i32p, _c_i32p]
    L.bc_pipeline_dev_status.restype = ctypes.c_int
    L.bc_pipeline_dev_trace.argtypes = [vp, _c_i32p, i32]
    L.bc_pipeline_dev_trace.restype = ctypes.c_int
    L.bc_pipeline_dev_read_plan.argtypes = [vp, ctypes.POINTER(BcDevPlan)]
    L.bc_pipeline_dev_read_plan.restype = ctypes.c_int
    _lib = L
    return L


def bc_status_str(status):
    return lib().bc_status_str(int(status)).decode()


# ---------------------------------------------------------------- marshalling
_DT = {torch.float32: BC_F32, torch.bfloat16: BC_BF16}


def _dev(t, name, dtype=None, numel=None, allow_none=False):
    """Device pointer of a contiguous CUDA tensor, after checks."""
    if t is None:
        if allow_none:
            return None
        raise ValueError("%s is required" % name)
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError("%s must be a CUDA tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if numel is not None and t.numel() < numel:
        raise ValueError("%s holds %d elements, needs %d" % (name, t.numel(), numel))
    return t.data_ptr()


def _host_i32(x):
    arr = np.ascontiguousarray(np.asarray(x, dtype=np.int32))
    return arr, arr.ctypes.data_as(_c_i32p)


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


class KVCache:
    """K and V tensors [n_seq][n_kv_heads][capacity][head_dim] of one dtype."""

    def __init__(self, k, v):
        if k.shape != v.shape or k.dtype != v.dtype or k.dim() != 4:
            raise ValueError("k and v must be [S][Hkv][cap][D] of one dtype")
        if k.dtype not in _DT:
            raise ValueError("cache dtype must be float32 or bfloat16")
        self.k, self.v = k, v
        self.n_seq, self.n_kv_heads, self.capacity, self.head_dim = (int(x) for x in k.shape)
        self.dtype = _DT[k.dtype]

    def struct(self):
        return BcKvCache(_dev(self.k, "cache.k"), _dev(self.v, "cache.v"), self.dtype, self.n_seq,
                         self.n_kv_heads, self.head_dim, self.capacity)

    def shape_struct(self):
        """Struct for workspace queries (no device pointers needed)."""
        return BcKvCache(1, 1, self.dtype, self.n_seq, self.n_kv_heads, self.head_dim, self.capacity)


def _active(q, k, v, blk_off, tdtype, Hkv, D, pointers=True):
    S, R, Hq, Dq = (int(x) for x in q.shape)
    if Dq != D:
        raise ValueError("q head_dim %d != cache head_dim %d" % (Dq, D))
    off_arr, off_p = _host_i32(blk_off)
    if pointers:
        qp = _dev(q, "q", tdtype, S * R * Hq * D)
        kp = _dev(k, "k", tdtype, S * Hkv * R * D)
        vp = _dev(v, "v", tdtype, S * Hkv * R * D)
    else:
        qp = kp = vp = 1
    act = BcActive(qp, kp, vp, off_p, len(off_arr) - 1, S, R, Hq)
    return act, off_arr


def bc_attn_workspace_bytes(prefix, priv, q_shape, blk_off, n_prefix_splits=0):
    """Workspace bytes for an attention call with these shapes (q_shape =
    (S, R, Hq, D)) and the caches' capacities."""
    S, R, Hq, D = q_shape
    off_arr, off_p = _host_i32(blk_off)
    act = BcActive(1, 1, 1, off_p, len(off_arr) - 1, S, R, Hq)
    ps = prefix.shape_struct()
    vs = priv.shape_struct() if priv is not None else None
    return int(lib().bc_attn_workspace_bytes(ctypes.byref(ps), ctypes.byref(vs) if vs else None,
                                             ctypes.byref(act), int(n_prefix_splits)))


def _attn_args(prefix, prefix_len, priv, priv_len, q, k, v, blk_off, mask, scale, out, ws, n_prefix_splits, stream):
    """Checked ctypes arguments of an attention call, and the host objects
    they point into (kept alive with them)."""
    tdtype = prefix.k.dtype
    act, off_arr = _active(q, k, v, blk_off, tdtype, prefix.n_kv_heads, prefix.head_dim)
    pl_arr, pl_p = _host_i32(prefix_len)
    if len(pl_arr) != prefix.n_seq:
        raise ValueError("prefix_len needs one entry per prefix sequence")
    ps = prefix.struct()
    if priv is not None:
        vs = priv.struct()
        vl_arr, vl_p = _host_i32(priv_len)
        if len(vl_arr) != act.n_seq:
            raise ValueError("priv_len needs one entry per rollout")
    else:
        vs, vl_arr, vl_p = None, None, None
    _dev(out, "out", tdtype, q.numel())
    args = (ctypes.byref(ps), pl_p, ctypes.byref(vs) if vs else None, vl_p, ctypes.byref(act), int(mask),
            float(scale), int(n_prefix_splits), out.data_ptr(), _dev(ws, "ws", torch.uint8), ws.numel(),
            _stream(stream))
    return args, (act, off_arr, pl_arr, ps, vs, vl_arr)


def _attn_call(name, prefix, prefix_len, priv, priv_len, q, k, v, blk_off, mask, scale, out, ws,
               n_prefix_splits, stream, check):
    args, _keep = _attn_args(prefix, prefix_len, priv, priv_len, q, k, v, blk_off, mask, scale, out, ws,
                             n_prefix_splits, stream)
    st = getattr(lib(), name)(*args)
    if check and st != BC_OK:
        raise BcError(st, name)
    return st


class Prepared:
    """One library call whose arguments were checked and marshalled once.
    Calling it issues the same call again: the same device pointers, and host
    arrays read afresh at each call (so an int32 length array updated in
    place by bc_kv_commit is seen).  The tensors and arrays it was made from
    must stay alive and keep their storage."""

    def __init__(self, name, args, keep):
        self.name, self.args, self._keep = name, args, keep
        self.fn = getattr(lib(), name)

    def __call__(self):
        st = self.fn(*self.args)
        if st != BC_OK:
            raise BcError(st, self.name)


def prepare_attn_step(prefix, prefix_len, priv, priv_len, q, k, v, blk_off, mask, scale, out, ws,
                      n_prefix_splits=0, stream=None):
    """bc_attn_step as a Prepared call; prefix_len must be a contiguous int32
    NumPy array (its current contents are passed at each call)."""
    if not (isinstance(prefix_len, np.ndarray) and prefix_len.dtype == np.int32 and prefix_len.flags.c_contiguous):
        raise ValueError("prefix_len must be a contiguous int32 NumPy array")
    args, keep = _attn_args(prefix, prefix_len, priv, priv_len, q, k, v, blk_off, mask, scale, out, ws,
                            n_prefix_splits, stream)
    return Prepared("bc_attn_step", args, keep + (prefix_len,))


def bc_attn_step(prefix, prefix_len, priv, priv_len, q, k, v, blk_off, mask, scale, out, ws,
                 n_prefix_splits=0, stream=None, check=True):
    return _attn_call("bc_attn_step", prefix, prefix_len, priv, priv_len, q, k, v, blk_off, mask, scale, out,
                      ws, n_prefix_splits, stream, check)


def bc_attn_partial(prefix, prefix_len, priv, priv_len, q, k, v, blk_off, mask, scale, out, ws,
                    n_prefix_splits=0, stream=None, check=True):
    return _attn_call("bc_attn_partial", prefix, prefix_len, priv, priv_len, q, k, v, blk_off, mask, scale,
                      out, ws, n_prefix_splits, stream, check)


def bc_attn_combine(prefix, prefix_len, priv, priv_len, q, k, v, blk_off, mask, scale, out, ws,
                    n_prefix_splits=0, stream=None, check=True):
    return _attn_call("bc_attn_combine", prefix, prefix_len, priv, priv_len, q, k, v, blk_off, mask, scale,
                      out, ws, n_prefix_splits, stream, check)


def bc_attn_step_static(prefix, prefix_len, priv, priv_len, q, k, v, blk_off, mask, scale, out,
                        n_prefix_splits=0, stream=None, check=True):
    """bc_attn_step without a workspace: the library's static scratch holds
    the split partials (nothing is allocated)."""
    tdtype = prefix.k.dtype
    act, _off = _active(q, k, v, blk_off, tdtype, prefix.n_kv_heads, prefix.head_dim)
    pl_arr, pl_p = _host_i32(prefix_len)
    if len(pl_arr) != prefix.n_seq:
        raise ValueError("prefix_len needs one entry per prefix sequence")
    ps = prefix.struct()
    vs, vl_arr, vl_p = None, None, None
    if priv is not None:
        vs = priv.struct()
        vl_arr, vl_p = _host_i32(priv_len)
        if len(vl_arr) != act.n_seq:
            raise ValueError("priv_len needs one entry per rollout")
    _dev(out, "out", tdtype, q.numel())
    st = lib().bc_attn_step_static(ctypes.byref(ps), pl_p, ctypes.byref(vs) if vs else None, vl_p,
                                   ctypes.byref(act), int(mask), float(scale), int(n_prefix_splits),
                                   out.data_ptr(), _stream(stream))
    if check and st != BC_OK:
        raise BcError(st, "bc_attn_step_static")
    return st


def bc_kv_commit(cache, length, seq, start, n_rows, blk_k, blk_v, stream=None, check=True):
    """``length`` is a host int32 NumPy array [n_seq], updated in place.
    seq = BC_ALL_SEQ commits blk_k / blk_v [n_seq][Hkv][n_rows][D] to every
    sequence."""
    if not (isinstance(length, np.ndarray) and length.dtype == np.int32 and length.flags.c_contiguous):
        raise ValueError("length must be a contiguous int32 NumPy array")
    if len(length) != cache.n_seq:
        raise ValueError("length needs one entry per sequence")
    n = cache.n_kv_heads * int(n_rows) * cache.head_dim * (cache.n_seq if seq == BC_ALL_SEQ else 1)
    kp = _dev(blk_k, "blk_k", cache.k.dtype, n)
    vp = _dev(blk_v, "blk_v", cache.k.dtype, n)
    cs = cache.struct()
    st = lib().bc_kv_commit(ctypes.byref(cs), length.ctypes.data_as(_c_i32p), int(seq), int(start),
                            int(n_rows), kp, vp, _stream(stream))
    if check and st != BC_OK:
        raise BcError(st, "bc_kv_commit")
    return st


def bc_unmask_workspace_bytes(n_rows, vocab):
    return int(lib().bc_unmask_workspace_bytes(int(n_rows), int(vocab)))


def bc_vocab_scan(logits, row_mask, with_sum, ws, stream=None, check=True):
    R, V = (int(x) for x in logits.shape)
    st = lib().bc_vocab_scan(_dev(logits, "logits", torch.float32, R * V), R, V,
                             _dev(row_mask, "row_mask", torch.uint8, R, allow_none=True), int(bool(with_sum)),
                             _dev(ws, "ws", torch.uint8), ws.numel(), _stream(stream))
    if check and st != BC_OK:
        raise BcError(st, "bc_vocab_scan")
    return st


def bc_unmask_select(logits, blk_off, mode, n_div, threshold, masked, tokens, conf, n_commit, ws,
                     stream=None, check=True):
    return _unmask_call("bc_unmask_select", logits, blk_off, mode, n_div, threshold, masked, tokens, conf,
                        n_commit, ws, stream, check)


def bc_unmask_decide(logits, blk_off, mode, n_div, threshold, masked, tokens, conf, n_commit, ws,
                     stream=None, check=True):
    return _unmask_call("bc_unmask_decide", logits, blk_off, mode, n_div, threshold, masked, tokens, conf,
                        n_commit, ws, stream, check)


def _unmask_args(logits, blk_off, mode, n_div, threshold, masked, tokens, conf, n_commit, ws, stream):
    R, V = (int(x) for x in logits.shape)
    off_arr, off_p = _host_i32(blk_off)
    n_blk = len(off_arr) - 1
    mode_arr, mode_p = _host_i32(mode)
    div_arr, div_p = _host_i32(n_div)
    if len(mode_arr) != n_blk or len(div_arr) != n_blk:
        raise ValueError("mode and n_div need one entry per block")
    args = (_dev(logits, "logits", torch.float32, R * V), R, V, off_p, n_blk, mode_p, div_p, float(threshold),
            _dev(masked, "masked", torch.uint8, R), _dev(tokens, "tokens", torch.int32, R),
            _dev(conf, "conf", torch.float32, R, allow_none=True), _dev(n_commit, "n_commit", torch.int32, n_blk),
            _dev(ws, "ws", torch.uint8), ws.numel(), _stream(stream))
    return args, (off_arr, mode_arr, div_arr)


def _unmask_call(name, logits, blk_off, mode, n_div, threshold, masked, tokens, conf, n_commit, ws,
                 stream, check):
    args, _keep = _unmask_args(logits, blk_off, mode, n_div, threshold, masked, tokens, conf, n_commit, ws, stream)
    st = getattr(lib(), name)(*args)
    if check and st != BC_OK:
        raise BcError(st, name)
    return st


def prepare_unmask_select(logits, blk_off, mode, n_div, threshold, masked, tokens, conf, n_commit, ws,
                          stream=None):
    """bc_unmask_select as a Prepared call."""
    args, keep = _unmask_args(logits, blk_off, mode, n_div, threshold, masked, tokens, conf, n_commit, ws, stream)
    return Prepared("bc_unmask_select", args, keep)


def bc_verify_workspace_bytes(n_seq, n_lrows, vocab):
    return int(lib().bc_verify_workspace_bytes(int(n_seq), int(n_lrows), int(vocab)))


def bc_spec_verify_sampled(logits, noise, inv_temperature, draft, fixed, first, accept_len, bonus, ws,
                           stream=None, check=True):
    S, L, V = (int(x) for x in logits.shape)
    m = int(draft.shape[1])
    st = lib().bc_spec_verify_sampled(
        _dev(logits, "logits", torch.float32, S * L * V), _dev(noise, "noise", torch.float32, S * L * V),
        ctypes.c_float(inv_temperature), S, L, V, _dev(draft, "draft", torch.int32, S * m), m,
        _dev(fixed, "fixed", torch.uint8, S * m, allow_none=True), _dev(first, "first", torch.int32, S),
        _dev(accept_len, "accept_len", torch.int32, S), _dev(bonus, "bonus", torch.int32, S),
        _dev(ws, "ws", torch.uint8), ws.numel(), _stream(stream))
    if check and st != BC_OK:
        raise BcError(st, "bc_spec_verify_sampled")
    return st


def _verify_args(logits, draft, fixed, first, accept_len, bonus, ws, stream):
    S, L, V = (int(x) for x in logits.shape)
    m = int(draft.shape[1])
    return (_dev(logits, "logits", torch.float32, S * L * V), S, L, V, _dev(draft, "draft", torch.int32, S * m), m,
            _dev(fixed, "fixed", torch.uint8, S * m, allow_none=True), _dev(first, "first", torch.int32, S),
            _dev(accept_len, "accept_len", torch.int32, S), _dev(bonus, "bonus", torch.int32, S),
            _dev(ws, "ws", torch.uint8), ws.numel(), _stream(stream))


def bc_spec_verify(logits, draft, fixed, first, accept_len, bonus, ws, stream=None, check=True):
    st = lib().bc_spec_verify(*_verify_args(logits, draft, fixed, first, accept_len, bonus, ws, stream))
    if check and st != BC_OK:
        raise BcError(st, "bc_spec_verify")
    return st


def prepare_spec_verify(logits, draft, fixed, first, accept_len, bonus, ws, stream=None):
    """bc_spec_verify as a Prepared call."""
    return Prepared("bc_spec_verify", _verify_args(logits, draft, fixed, first, accept_len, bonus, ws, stream),
                    (logits, draft, fixed, first, accept_len, bonus, ws))


class Pipeline:
    """The pipelined parallel decoding schedule (bc_pipeline_*): a host state
    machine, no GPU involved.  plan() returns the next step's (active blocks,
    local steps, modes, n_div, blk_off, row0), or None when every block is
    committed; report(n_commit) returns the blocks to commit, in order."""

    def __init__(self, block_sizes, window, add, act, n_div):
        sizes = np.ascontiguousarray(np.asarray(block_sizes, dtype=np.int32))
        h = ctypes.c_void_p()
        st = lib().bc_pipeline_create(sizes.ctypes.data_as(_c_i32p), len(sizes), int(window), float(add),
                                      float(act), int(n_div), ctypes.byref(h))
        if st != BC_OK:
            raise BcError(st, "bc_pipeline_create")
        self._h = h
        self.window = int(window)
        w = self.window
        self._active, self._local, self._mode, self._div = (np.zeros(w, np.int32) for _ in range(4))
        self._off = np.zeros(w + 1, np.int32)
        self._row0 = np.zeros(1, np.int32)
        self._done = np.zeros(w, np.int32)
        self._counts = np.zeros(w, np.int32)
        p = lambda a: a.ctypes.data_as(_c_i32p)
        self._next_args = (h, p(self._active), p(self._local), p(self._mode), p(self._div), p(self._off),
                           p(self._row0))

    def plan(self):
        n = lib().bc_pipeline_next(*self._next_args)
        if n < 0:
            raise BcError(n, "bc_pipeline_next")
        if n == 0:
            return None
        return (self._active[:n].tolist(), self._local[:n].tolist(), self._mode[:n].tolist(),
                self._div[:n].tolist(), self._off[:n + 1].tolist(), int(self._row0[0]))

    def report(self, n_commit):
        c = np.ascontiguousarray(np.asarray(n_commit, dtype=np.int32))
        k = lib().bc_pipeline_report(self._h, c.ctypes.data_as(_c_i32p), self._done.ctypes.data_as(_c_i32p))
        if k < 0:
            raise BcError(k, "bc_pipeline_report")
        return self._done[:k].tolist()

    def decode(self, cache, length, n_q_heads, vocab, scale, threshold, masked, tokens, out, ws_attn, ws_unmask,
               inputs, after_attn=None, max_steps=4096, stream=None):
        """bc_pipeline_decode: the whole step loop in the library.

        inputs(step, active, local_steps) returns the step's BcStepInputs
        (device pointers kept alive by the caller); after_attn(step, active,
        local_steps, cache_len, out_ptr) is optional.  ``length`` is the host
        int32 cache length [1], advanced in place.  Returns (n_steps, trace)
        with the trace as a list of dicts (active, modes, n_commit,
        committed), like a step-by-step decode records it."""
        if not (isinstance(length, np.ndarray) and length.dtype == np.int32 and length.flags.c_contiguous):
            raise ValueError("length must be a contiguous int32 NumPy array")
        if cache.n_seq != 1 or len(length) != 1:
            raise ValueError("the pipelined decode runs one sequence")
        w = self.window
        stride = pipe_trace_ints(w)
        trace = np.full((int(max_steps), stride), -1, np.int32)
        n_steps = np.zeros(1, np.int32)
        errors = []

        def _inputs(user, step, n, active, local, dst):
            try:
                src = inputs(int(step), [active[j] for j in range(n)], [local[j] for j in range(n)])
                ctypes.memmove(dst, ctypes.addressof(src), ctypes.sizeof(BcStepInputs))
                return 0
            except BaseException as e:   # noqa: BLE001 -- re-raised after the call
                errors.append(e)
                return 1

        def _after(user, step, n, active, local, cache_len, outp):
            try:
                after_attn(int(step), [active[j] for j in range(n)], [local[j] for j in range(n)], int(cache_len),
                           outp)
                return 0
            except BaseException as e:   # noqa: BLE001
                errors.append(e)
                return 1

        fi = STEP_INPUTS_FN(_inputs)
        fa = AFTER_ATTN_FN(_after) if after_attn is not None else AFTER_ATTN_FN()
        cs = cache.struct()
        st = lib().bc_pipeline_decode(
            self._h, ctypes.byref(cs), length.ctypes.data_as(_c_i32p), int(n_q_heads), int(vocab), float(scale),
            float(threshold), _dev(masked, "masked", torch.uint8), _dev(tokens, "tokens", torch.int32),
            _dev(out, "out"), _dev(ws_attn, "ws_attn"), ws_attn.numel() * ws_attn.element_size(),
            _dev(ws_unmask, "ws_unmask"), ws_unmask.numel() * ws_unmask.element_size(), fi, fa, None,
            trace.ctypes.data_as(_c_i32p), int(max_steps), n_steps.ctypes.data_as(_c_i32p), _stream(stream))
        if errors:
            raise errors[0]
        if st != BC_OK:
            raise BcError(st, "bc_pipeline_decode")
        k = int(n_steps[0])
        rows = trace[:k].tolist()
        recs = []
        for r in rows:
            n, nd = r[0], r[1]
            recs.append(dict(active=r[2:2 + n], modes=["full" if m == BC_UNMASK_FULL else "semi" for m in r[2 + w:2 + w + n]],
                             n_commit=r[2 + 2 * w:2 + 2 * w + n], committed=r[2 + 3 * w:2 + 3 * w + nd]))
        return k, recs

    def close(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.bc_pipeline_destroy(h)
        self._h = None

    def __del__(self):
        self.close()


class DevicePipeline:
    """The pipelined decode with the schedule on the device
    (bc_pipeline_dev_*): the library's device state, workspaces and trace;
    the caller's step buffers (R rows, R = ``rows``), cache and
    masked / tokens.  ``step`` enqueues one step and reads nothing back, so
    steps can be captured in a graph; ``status`` reads the mapped state once
    the stream has run."""

    def __init__(self, block_sizes, window, add, act, n_div, cache, prefix_len, n_q_heads, vocab, scale, threshold,
                 masked, tokens, q, k, v, logits, out, max_steps):
        sizes = np.ascontiguousarray(np.asarray(block_sizes, dtype=np.int32))
        h = ctypes.c_void_p()
        cs = cache.struct()
        st = lib().bc_pipeline_dev_create(
            sizes.ctypes.data_as(_c_i32p), len(sizes), int(window), float(add), float(act), int(n_div),
            ctypes.byref(cs), int(prefix_len), int(n_q_heads), int(vocab), float(scale), float(threshold),
            _dev(masked, "masked", torch.uint8), _dev(tokens, "tokens", torch.int32), _dev(q, "q"), _dev(k, "k"),
            _dev(v, "v"), _dev(logits, "logits", torch.float32), _dev(out, "out"), int(max_steps), ctypes.byref(h))
        if st != BC_OK:
            raise BcError(st, "bc_pipeline_dev_create")
        self._h = h
        self.window = int(window)
        self.max_steps = int(max_steps)
        self.rows = int(lib().bc_pipeline_dev_rows(h))
        self._keep = (cache, masked, tokens, q, k, v, logits, out)

    def plan_ptr(self):
        return int(lib().bc_pipeline_dev_plan(self._h))

    def read_plan(self):
        """The next step's plan, copied to the host (synchronous)."""
        p = BcDevPlan()
        st = lib().bc_pipeline_dev_read_plan(self._h, ctypes.byref(p))
        if st != BC_OK:
            raise BcError(st, "bc_pipeline_dev_read_plan")
        return p

    def reset(self, stream=None):
        st = lib().bc_pipeline_dev_reset(self._h, _stream(stream))
        if st != BC_OK:
            raise BcError(st, "bc_pipeline_dev_reset")

    def step(self, stream=None):
        st = lib().bc_pipeline_dev_step(self._h, _stream(stream))
        if st != BC_OK:
            raise BcError(st, "bc_pipeline_dev_step")

    def replay(self, table, max_local, stream=None):
        """``table``: a device uint8 tensor holding BcStepBlock entries
        [n_blocks][max_local]."""
        st = lib().bc_pipeline_dev_replay(self._h, _dev(table, "table", torch.uint8), int(max_local),
                                          _stream(stream))
        if st != BC_OK:
            raise BcError(st, "bc_pipeline_dev_replay")

    def status(self):
        """(finished, steps, cache length, error) after the enqueued work has run."""
        vals = [ctypes.c_int32() for _ in range(4)]
        lib().bc_pipeline_dev_status(self._h, *[ctypes.byref(x) for x in vals])
        return tuple(int(x.value) for x in vals)

    def trace(self):
        """The steps run, as bc_pipeline_decode's trace records (synchronous)."""
        w = self.window
        buf = np.full((self.max_steps, pipe_trace_ints(w)), -1, np.int32)
        k = lib().bc_pipeline_dev_trace(self._h, buf.ctypes.data_as(_c_i32p), self.max_steps)
        if k < 0:
            raise BcError(k, "bc_pipeline_dev_trace")
        recs = []
        for r in buf[:k].tolist():
            n, nd = r[0], r[1]
            recs.append(dict(active=r[2:2 + n], modes=["full" if m == BC_UNMASK_FULL else "semi" for m in r[2 + w:2 + w + n]],
                             n_commit=r[2 + 2 * w:2 + 2 * w + n], committed=r[2 + 3 * w:2 + 3 * w + nd]))
        return recs

    def close(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.bc_pipeline_dev_destroy(h)
        self._h = None

    def __del__(self):
        self.close()
