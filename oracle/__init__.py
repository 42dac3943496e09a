"""CPU oracle for the block-diffusion denoise step (fp64, plain loops).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package; the GPU library and
its Python binding never do, and the two share no code.

The arithmetic lives in ``bd_oracle.c`` (compiled with gcc, no fast-math);
this module only builds it, loads it with ctypes and marshals numpy arrays.
Each wrapper names the passage its C function follows.
"""

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bd_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16, FP8 = 0, 1, 2
BIDIR, CAUSAL, QUAD = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP over independent query rows, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        # Build on first use, and again whenever the source is newer than the library.
        if not os.path.exists(_LIB) or os.path.getmtime(_SRC) > os.path.getmtime(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32 = ctypes.c_int
        lib.bdo_attention.argtypes = [i32] * 8 + [ctypes.c_double] + [P] * 7
        lib.bdo_attention.restype = None
        lib.bdo_confidence_row.argtypes = [i32, P, P, P, P, P]
        lib.bdo_commit_k.argtypes = [i32, i32, i32]
        lib.bdo_commit_k.restype = i32
        lib.bdo_confidence_commit.argtypes = [i32, i32, i32, i32, ctypes.c_double] + [P] * 7
        lib.bdo_spec_verify.argtypes = [i32, i32, i32, P, P, P, P]
        lib.bdo_kv_append.argtypes = [i32] * 6 + [P] * 7
        lib.bdo_num_threads.restype = i32
        lib.bdo_set_num_threads.argtypes = [i32]
        lib.bdo_softmax_partial.argtypes = [i32, i32, P, P, P, P, P]
        lib.bdo_merge_partials.argtypes = [i32, i32, P, P, P, P]
        lib.bdo_lm_head_logits.argtypes = [i32, i32, i32, P, P, P]
        lib.bdo_attention_fp8kv.argtypes = [i32] * 7 + [ctypes.c_double] + [P] * 9
        lib.bdo_fp8_e4m3_decode.argtypes = [i32, P, P]
        lib.bdo_attention_quad.argtypes = [i32] * 7 + [ctypes.c_double] + [P] * 7
        lib.bdo_attention_quad_fp8kv.argtypes = [i32] * 6 + [ctypes.c_double] + [P] * 9
        lib.bdo_two_stream_attention.argtypes = [i32] * 9 + [ctypes.c_double, i32] + [P] * 6
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    assert a.dtype == dtype, (a.dtype, dtype)
    return a


def num_threads() -> int:
    return int(_load().bdo_num_threads())


def set_num_threads(n: int) -> None:
    """Threads the oracle's parallel loops (independent query rows) use from now on."""
    _load().bdo_set_num_threads(int(n))


def attention(q, k_blk, v_blk, k_cache, v_cache, prefix, mode, scale=None):
    """Block attention of Fast-dVLM's causal-context decoding (Fast-dVLM write-up,
    sections 4.1 and 5.3; summary page Fig. 3): returns float64 [n][D][Hq][d]."""
    lib = _load()
    n, D, Hq, d = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    dtype = F32 if q.dtype == np.float32 else BF16
    el = np.float32 if dtype == F32 else np.uint16
    arrs = [_c(a, el) for a in (q, k_blk, v_blk, k_cache, v_cache)]
    assert k_blk.shape == (n, D, Hkv, d) and v_blk.shape == (n, D, Hkv, d)
    assert k_cache.shape == (n, Hkv, cap, d) and v_cache.shape == (n, Hkv, cap, d)
    prefix = _c(prefix, np.int32)
    assert prefix.shape == (n,) and np.all(prefix >= 0) and np.all(prefix <= cap)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((n, D, Hq, d), dtype=np.float64)
    lib.bdo_attention(n, D, Hq, Hkv, d, cap, dtype, int(mode), float(scale),
                      *[_ptr(a) for a in arrs], _ptr(prefix), _ptr(out))
    return out


def confidence_row(x):
    """Confidence and greedy token of one logits row (DiffusionVL notes, cached block
    decoding: confidence = model probability of the chosen token).
    Returns (conf, argmax, lse, p2) with conf, lse, p2 in float64."""
    lib = _load()
    x = _c(x, np.float32)
    conf, lse, p2 = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    a = ctypes.c_int32()
    lib.bdo_confidence_row(x.size, _ptr(x), ctypes.byref(conf), ctypes.byref(a),
                           ctypes.byref(lse), ctypes.byref(p2))
    return conf.value, a.value, lse.value, p2.value


def commit_k(D, S, n_masked):
    """k = min(ceil(D/S), |M|) (DiffusionVL notes, Algorithm 1)."""
    return int(_load().bdo_commit_k(int(D), int(S), int(n_masked)))


def confidence_commit(logits, masked, tokens, S, tau):
    """One denoising step's confidence + dynamic commit (DiffusionVL notes, cached
    block decoding and Algorithm 1).  ``masked`` and ``tokens`` are updated in place
    (copies are returned too).  Returns dict(conf, argmax, committed, n_committed,
    masked, tokens)."""
    lib = _load()
    n_req, D, V = logits.shape
    logits = _c(logits, np.float32)
    masked = np.array(masked, dtype=np.uint8, copy=True, order="C")
    tokens = np.array(tokens, dtype=np.int32, copy=True, order="C")
    conf = np.zeros((n_req, D), np.float64)
    amax = np.zeros((n_req, D), np.int32)
    committed = np.zeros((n_req, D), np.uint8)
    ncom = np.zeros(n_req, np.int32)
    lib.bdo_confidence_commit(n_req, D, V, int(S), float(tau), _ptr(logits), _ptr(masked),
                              _ptr(tokens), _ptr(conf), _ptr(amax), _ptr(committed), _ptr(ncom))
    return dict(conf=conf, argmax=amax, committed=committed, n_committed=ncom,
                masked=masked, tokens=tokens)


def spec_verify(logits, draft):
    """Longest accepted draft prefix (Fast-dVLM write-up, section 5.3, linear
    speculative decoding).  Returns (accepted_len int32[n_req], argmax int32[n_req][D])."""
    lib = _load()
    n_req, D, V = logits.shape
    logits = _c(logits, np.float32)
    draft = _c(draft, np.int32)
    L = np.zeros(n_req, np.int32)
    amax = np.zeros((n_req, D), np.int32)
    lib.bdo_spec_verify(n_req, D, V, _ptr(logits), _ptr(draft), _ptr(L), _ptr(amax))
    return L, amax


def kv_append(k_cache, v_cache, prefix, k_blk, v_blk, n_accept=None):
    """Append accepted block K/V to the cache (Fast-dVLM write-up, section 5.3: crop
    the cache to the accepted prefix; DiffusionVL notes: a finished block joins the
    history cache).  Element type from k_cache: float32, bf16 bits (uint16) or E4M3
    bytes (uint8).  Returns new (k_cache, v_cache, prefix, err)."""
    lib = _load()
    n, Hkv, cap, d = k_cache.shape
    D = k_blk.shape[1]
    dtype = {np.dtype(np.float32): F32, np.dtype(np.uint16): BF16, np.dtype(np.uint8): FP8}[k_cache.dtype]
    k_cache = np.array(k_cache, copy=True, order="C")
    v_cache = np.array(v_cache, copy=True, order="C")
    prefix = np.array(prefix, dtype=np.int32, copy=True)
    kb = np.ascontiguousarray(k_blk)
    vb = np.ascontiguousarray(v_blk)
    na = None if n_accept is None else _c(n_accept, np.int32)
    err = np.zeros(1, np.int32)
    lib.bdo_kv_append(n, D, Hkv, d, cap, dtype, _ptr(k_cache), _ptr(v_cache), _ptr(prefix),
                      _ptr(kb), _ptr(vb), _ptr(na), _ptr(err))
    return k_cache, v_cache, prefix, int(err[0])


def softmax_partial(s, v):
    """Split-K partial of one key range (online softmax normaliser, Milakov and
    Gimelshein 2018): returns (m, l, o) with m = max s, l = sum exp(s - m) and o
    the range's normalised weighted value sum.  s: [nk], v: [nk][d]."""
    lib = _load()
    s = _c(s, np.float64)
    v = _c(v, np.float64)
    nk, d = v.shape
    m = ctypes.c_double()
    l = ctypes.c_double()
    o = np.zeros(d, np.float64)
    lib.bdo_softmax_partial(nk, d, _ptr(s), _ptr(v), ctypes.byref(m), ctypes.byref(l), _ptr(o))
    return m.value, l.value, o


def merge_partials(parts):
    """Merge split-K partials in the given order: M = max m_p, c_p = exp(m_p - M) l_p,
    out = sum c_p o_p / sum c_p (the same source).  parts: list of (m, l, o)."""
    lib = _load()
    m = np.array([p[0] for p in parts], np.float64)
    l = np.array([p[1] for p in parts], np.float64)
    o = np.ascontiguousarray(np.stack([p[2] for p in parts]).astype(np.float64))
    out = np.zeros(o.shape[1], np.float64)
    lib.bdo_merge_partials(len(parts), o.shape[1], _ptr(m), _ptr(l), _ptr(o), _ptr(out))
    return out


def lm_head_logits(hidden, weight):
    """Logits of every block slot: the vocabulary projection of its final hidden
    state, logits[r][i][v] = sum_h hidden[r][i][h] * weight[v][h], in fp64.
    hidden: raw bf16 [n_req][D][H]; weight: raw bf16 [V][H].  Their softmax is the
    distribution whose top probability is the confidence (DiffusionVL notes,
    cached block decoding)."""
    lib = _load()
    n_req, D, H = hidden.shape
    V = weight.shape[0]
    h = _c(hidden, np.uint16)
    w = _c(weight, np.uint16)
    out = np.zeros((n_req, D, V), np.float64)
    lib.bdo_lm_head_logits(n_req * D, V, H, _ptr(h), _ptr(w), _ptr(out))
    return out


def attention_fp8kv(q, k_blk, v_blk, k_cache, v_cache, k_scale, v_scale, prefix, mode, scale=None, B=None):
    """Block attention with an FP8 KV cache (the same mask rules as attention(), or
    attention_quad()'s when mode is QUAD with draft block size B):
    q raw bf16; k_blk, v_blk, k_cache, v_cache raw OCP E4M3 bytes in the same
    layouts; every key / value is its byte's E4M3 value times the fp32 scale of its
    (item, KV head), k_scale / v_scale [n][Hkv].  Returns fp64 [n][slots][Hq][d]."""
    lib = _load()
    n, D, Hq, d = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    q = _c(q, np.uint16)
    kb, vb = _c(k_blk, np.uint8), _c(v_blk, np.uint8)
    kc, vc = _c(k_cache, np.uint8), _c(v_cache, np.uint8)
    ks, vs = _c(k_scale, np.float32), _c(v_scale, np.float32)
    pre = _c(prefix, np.int32)
    out = np.zeros((n, D, Hq, d), np.float64)
    if mode == QUAD:
        assert D == quad_slots(B), (D, B)
        lib.bdo_attention_quad_fp8kv(n, int(B), Hq, Hkv, d, cap, float(scale), _ptr(q), _ptr(kb), _ptr(vb),
                                     _ptr(kc), _ptr(vc), _ptr(ks), _ptr(vs), _ptr(pre), _ptr(out))
        return out
    lib.bdo_attention_fp8kv(n, D, Hq, Hkv, d, cap, int(mode), float(scale), _ptr(q), _ptr(kb), _ptr(vb),
                            _ptr(kc), _ptr(vc), _ptr(ks), _ptr(vs), _ptr(pre), _ptr(out))
    return out


def quad_slots(B):
    """Block slots of a quadratic self-speculative step: B drafts, then B - g mask
    tokens for each group g = 0..B-1."""
    return B * (B + 3) // 2


def attention_quad(q, k_blk, v_blk, k_cache, v_cache, prefix, B, scale=None):
    """Quadratic self-speculative attention (Fast-dVLM write-up, section 5.3, the
    quadratic variant): block slots 0..B-1 are the draft tokens (causal among
    themselves), then group g's mask tokens (B - g slots) see the drafts before g
    and their own group.  Every slot sees the cache.  Layouts as attention() with
    quad_slots(B) block slots.  Returns float64 [n][quad_slots(B)][Hq][d]."""
    lib = _load()
    n, S, Hq, d = q.shape
    assert S == quad_slots(B), (S, B)
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    dtype = F32 if q.dtype == np.float32 else BF16
    el = np.float32 if dtype == F32 else np.uint16
    arrs = [_c(a, el) for a in (q, k_blk, v_blk, k_cache, v_cache)]
    prefix = _c(prefix, np.int32)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((n, S, Hq, d), dtype=np.float64)
    lib.bdo_attention_quad(n, int(B), Hq, Hkv, d, cap, dtype, float(scale), *[_ptr(a) for a in arrs],
                           _ptr(prefix), _ptr(out))
    return out


def two_stream_attention(q, k, v, spans, n_spans, Lc, D, scale=None):
    """Two-stream training attention (Fast-dVLM write-up, sections 4.1, 4.3, 4.4;
    summary page Fig. 3) over [clean stream ; noisy stream]: clean queries are
    causal over the clean stream; a noisy query sees the clean positions before its
    block and its own block of the noisy stream (bidirectional), blocks of D tokens
    cut from each response's start and truncated at its end.
    q [n][L][Hq][d] (L = Lc + Ln), k and v [n][Hkv][cap][d] (bf16 bits or fp32),
    spans int32 [n][max_spans][2] = (clean start, length) of each response,
    n_spans int32 [n].  Returns float64 [n][L][Hq][d]."""
    lib = _load()
    n, L, Hq, d = q.shape
    Hkv, cap = k.shape[1], k.shape[2]
    Ln = L - Lc
    dtype = F32 if q.dtype == np.float32 else BF16
    el = np.float32 if dtype == F32 else np.uint16
    q, k, v = _c(q, el), _c(k, el), _c(v, el)
    spans = _c(spans, np.int32)
    n_spans = _c(n_spans, np.int32)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((n, L, Hq, d), np.float64)
    lib.bdo_two_stream_attention(n, Lc, Ln, cap, D, Hq, Hkv, d, dtype, float(scale), spans.shape[1], _ptr(q),
                                 _ptr(k), _ptr(v), _ptr(spans), _ptr(n_spans), _ptr(out))
    return out


def fp8_e4m3_decode(b):
    """OCP FP8 E4M3 bytes -> fp64 (the decode the FP8-KV attention applies)."""
    lib = _load()
    b = _c(b, np.uint8)
    out = np.zeros(b.shape, np.float64)
    lib.bdo_fp8_e4m3_decode(b.size, _ptr(b), _ptr(out))
    return out
