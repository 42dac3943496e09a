"""Thin ctypes binding of libbd.so (the C ABI declared in include/bd.h).

Argument marshalling only: tensors are passed as raw device pointers, the
stream as torch's current HIP stream.  Every step of the computation runs in
the HIP kernels of libbd.so; if the library is missing this module raises on
import rather than falling back to anything else.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbd.so")

BD_OK, BD_E_NULL, BD_E_SHAPE, BD_E_DTYPE, BD_E_PARAM, BD_E_WORKSPACE, BD_E_LAUNCH, BD_E_SCRATCH = range(8)
BD_F32, BD_BF16, BD_FP8KV = 0, 1, 2
BD_BLOCK_BIDIR, BD_BLOCK_CAUSAL, BD_BLOCK_QUAD = 0, 1, 2
BD_PLAN_BALANCED = 0x100
SIZE_MAX = (1 << 64) - 1


class BdAttnDesc(ctypes.Structure):
    _fields_ = [("n_items", ctypes.c_int32), ("D", ctypes.c_int32), ("Hq", ctypes.c_int32),
                ("Hkv", ctypes.c_int32), ("d", ctypes.c_int32), ("cap", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("mode", ctypes.c_int32), ("max_prefix", ctypes.c_int32),
                ("scale", ctypes.c_float)]


class BdCommitDesc(ctypes.Structure):
    _fields_ = [("n_req", ctypes.c_int32), ("D", ctypes.c_int32), ("V", ctypes.c_int32),
                ("S", ctypes.c_int32), ("tau", ctypes.c_float)]


class BdLmheadDesc(ctypes.Structure):
    _fields_ = [("n_req", ctypes.c_int32), ("D", ctypes.c_int32), ("V", ctypes.c_int32),
                ("H", ctypes.c_int32), ("S", ctypes.c_int32), ("tau", ctypes.c_float)]


class BdTwoStreamDesc(ctypes.Structure):
    _fields_ = [("n_seq", ctypes.c_int32), ("Lc", ctypes.c_int32), ("Ln", ctypes.c_int32), ("cap", ctypes.c_int32),
                ("D", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("d", ctypes.c_int32),
                ("max_spans", ctypes.c_int32), ("scale", ctypes.c_float)]


class BdError(RuntimeError):
    def __init__(self, fn, status, lib):
        msg = lib.bd_status_string(status).decode()
        if status == BD_E_LAUNCH:
            msg += " (hipError %d)" % lib.bd_last_hip_error()
        super().__init__("%s failed: status %d: %s" % (fn, status, msg))
        self.status = status


def _load():
    # torch ships its own libamdhip64.so.7.  Load it first, so libbd.so binds to
    # the same HIP runtime that owns torch's device memory and streams (both
    # libraries carry the same soname; whichever loads first serves the process).
    import torch
    # Start that runtime before libbd.so is loaded.  Loading libbd.so registers
    # its code objects with the runtime and an exit handler that unregisters
    # them (hipcc's module constructor calls atexit); exit handlers run in the
    # reverse order of registration, so this one then runs before any handler
    # registered while the runtime started (a profiler's finalisation, say),
    # while the runtime is still whole.  On a machine without a GPU this only
    # reports that there is none.
    torch.cuda.is_available()
    if not os.path.exists(LIB_PATH):
        raise ImportError("libbd.so is not built (%s); run __graft_entry__.build() or "
                          "python vlm_decoding_amd/build.py" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    sz = ctypes.c_size_t
    i32 = ctypes.c_int32
    AD = ctypes.POINTER(BdAttnDesc)
    CD = ctypes.POINTER(BdCommitDesc)
    LD = ctypes.POINTER(BdLmheadDesc)
    TD = ctypes.POINTER(BdTwoStreamDesc)
    sig = {
        "bd_attn_workspace_bytes": (sz, [AD]),
        "bd_attn_step": (i32, [AD, P, P, P, P, P, P, P, P, sz, P]),
        "bd_attn_step_fp8kv": (i32, [AD, P, P, P, P, P, P, P, P, P, P, sz, P]),
        "bd_attn_step_noalloc": (i32, [AD, P, P, P, P, P, P, P, P]),
        "bd_attn_noalloc_max_scratch_bytes": (sz, []),
        "bd_commit_workspace_bytes": (sz, [CD]),
        "bd_confidence_commit": (i32, [CD, P, P, P, P, P, P, P, P, sz, P]),
        "bd_verify_workspace_bytes": (sz, [i32, i32, i32]),
        "bd_spec_verify": (i32, [i32, i32, i32, P, P, P, P, P, sz, P]),
        "bd_kv_append": (i32, [AD, P, P, P, P, P, P, P, P]),
        "bd_lmhead_workspace_bytes": (sz, [LD]),
        "bd_lmhead_confidence_commit": (i32, [LD, P, P, P, P, P, P, P, P, P, sz, P]),
        "bd_two_stream_workspace_bytes": (sz, [TD]),
        "bd_two_stream_attn": (i32, [TD, P, P, P, P, P, P, P, sz, P]),
        "bd_status_string": (ctypes.c_char_p, [i32]),
        "bd_last_hip_error": (i32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def _ptr(t):
    """Device pointer of a tensor (or None); raw ints pass through."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _check(fn, status):
    if status != BD_OK:
        raise BdError(fn, status, lib)


def attn_desc(n_items, D, Hq, Hkv, d, cap, dtype, mode, max_prefix, scale=None):
    return BdAttnDesc(n_items, D, Hq, Hkv, d, cap, dtype, mode, max_prefix,
                      (1.0 / d ** 0.5) if scale is None else scale)


def commit_desc(n_req, D, V, S, tau):
    return BdCommitDesc(n_req, D, V, S, tau)


def bd_attn_workspace_bytes(desc):
    return lib.bd_attn_workspace_bytes(ctypes.byref(desc))


def bd_attn_step(desc, q, k_blk, v_blk, k_cache, v_cache, prefix_len, out, workspace,
                 workspace_bytes=None, stream=None):
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("bd_attn_step", lib.bd_attn_step(
        ctypes.byref(desc), _ptr(q), _ptr(k_blk), _ptr(v_blk), _ptr(k_cache), _ptr(v_cache),
        _ptr(prefix_len), _ptr(out), _ptr(workspace), workspace_bytes, _stream(stream)))


def bd_attn_step_noalloc(desc, q, k_blk, v_blk, k_cache, v_cache, prefix_len, out, stream=None):
    _check("bd_attn_step_noalloc", lib.bd_attn_step_noalloc(
        ctypes.byref(desc), _ptr(q), _ptr(k_blk), _ptr(v_blk), _ptr(k_cache), _ptr(v_cache), _ptr(prefix_len),
        _ptr(out), _stream(stream)))


def bd_attn_step_fp8kv(desc, q, k_blk, v_blk, k_cache, v_cache, k_scale, v_scale, prefix_len, out,
                       workspace, workspace_bytes=None, stream=None):
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("bd_attn_step_fp8kv", lib.bd_attn_step_fp8kv(
        ctypes.byref(desc), _ptr(q), _ptr(k_blk), _ptr(v_blk), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
        _ptr(v_scale), _ptr(prefix_len), _ptr(out), _ptr(workspace), workspace_bytes, _stream(stream)))


def bd_commit_workspace_bytes(desc):
    return lib.bd_commit_workspace_bytes(ctypes.byref(desc))


def bd_confidence_commit(desc, logits, masked, tokens, conf=None, argmax=None, committed=None,
                         n_committed=None, workspace=None, workspace_bytes=None, stream=None):
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("bd_confidence_commit", lib.bd_confidence_commit(
        ctypes.byref(desc), _ptr(logits), _ptr(masked), _ptr(tokens), _ptr(conf), _ptr(argmax),
        _ptr(committed), _ptr(n_committed), _ptr(workspace), workspace_bytes, _stream(stream)))


def bd_verify_workspace_bytes(n_req, D, V):
    return lib.bd_verify_workspace_bytes(n_req, D, V)


def bd_spec_verify(n_req, D, V, logits, draft, accepted_len, argmax=None, workspace=None,
                   workspace_bytes=None, stream=None):
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("bd_spec_verify", lib.bd_spec_verify(
        n_req, D, V, _ptr(logits), _ptr(draft), _ptr(accepted_len), _ptr(argmax), _ptr(workspace),
        workspace_bytes, _stream(stream)))


def bd_kv_append(desc, k_cache, v_cache, prefix_len, k_blk, v_blk, n_accept=None, dev_err=None,
                 stream=None):
    _check("bd_kv_append", lib.bd_kv_append(
        ctypes.byref(desc), _ptr(k_cache), _ptr(v_cache), _ptr(prefix_len), _ptr(k_blk), _ptr(v_blk),
        _ptr(n_accept), _ptr(dev_err), _stream(stream)))


def lmhead_desc(n_req, D, V, H, S, tau):
    return BdLmheadDesc(n_req, D, V, H, S, tau)


def bd_lmhead_workspace_bytes(desc):
    return lib.bd_lmhead_workspace_bytes(ctypes.byref(desc))


def bd_lmhead_confidence_commit(desc, hidden, weight, masked, tokens, conf=None, argmax=None, committed=None,
                                n_committed=None, workspace=None, workspace_bytes=None, stream=None):
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("bd_lmhead_confidence_commit", lib.bd_lmhead_confidence_commit(
        ctypes.byref(desc), _ptr(hidden), _ptr(weight), _ptr(masked), _ptr(tokens), _ptr(conf), _ptr(argmax),
        _ptr(committed), _ptr(n_committed), _ptr(workspace), workspace_bytes, _stream(stream)))


def two_stream_desc(n_seq, Lc, Ln, cap, D, Hq, Hkv, d, max_spans, scale=None):
    return BdTwoStreamDesc(n_seq, Lc, Ln, cap, D, Hq, Hkv, d, max_spans, (1.0 / d ** 0.5) if scale is None else scale)


def bd_two_stream_workspace_bytes(desc):
    return lib.bd_two_stream_workspace_bytes(ctypes.byref(desc))


def bd_two_stream_attn(desc, q, k, v, spans, n_spans, out, workspace=None, workspace_bytes=None, stream=None):
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("bd_two_stream_attn", lib.bd_two_stream_attn(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(spans), _ptr(n_spans), _ptr(out), _ptr(workspace),
        workspace_bytes, _stream(stream)))
