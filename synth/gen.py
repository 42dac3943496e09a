"""Seeded synthetic inputs for one block-diffusion step.

This module draws numbers and lays them out in the byte layouts that the
C-ABI library and the CPU oracle both read.  It holds none of the step's
arithmetic (no attention, no softmax, no ranking): only random draws, the
bf16 rounding of those draws, placement in memory, and the planting of
chosen logit peaks.

Layouts (row-major, innermost last):

    q        [n][D][Hq][d]        this step's queries for every block slot
    k_blk    [n][D][Hkv][d]       this step's block keys
    v_blk    [n][D][Hkv][d]       this step's block values
    k_cache  [n][Hkv][cap][d]     frozen keys of the prompt and finished blocks
    v_cache  [n][Hkv][cap][d]     frozen values
    prefix   int32[n]             valid cache length per item
    logits   f32 [n_req][D][V]
    masked   u8  [n_req][D]       1 = still [MASK]
    tokens   i32 [n_req][D]       committed ids; -1 at masked slots
    draft    i32 [n_req][D]       draft ids to verify (speculative configs)

Cache slots at and beyond ``prefix`` are filled with NaN bit patterns, so
a kernel that reads past the valid prefix cannot go unnoticed.

Draw order for a step (one Generator(PCG64(seed)) per step): prefix
lengths, Q, K cache, V cache, block K, block V, the masked set, committed
token ids, logits, then plants.
"""

import numpy as np

from .configs import (BF16, CONFIGS, F32, FP8KV, LMHEAD_CONFIGS, QUAD, QUAD_CONFIGS, TWO_STREAM_CONFIGS,
                      lmhead_seed_of, quad_seed_of, seed_of, two_stream_seed_of)

BF16_NAN = np.uint16(0x7FC0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); return the raw 16-bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((b >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen raw bf16 patterns to float32 exactly."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# The non-negative finite OCP FP8 E4M3 values (exponent bias 7, 3 mantissa bits,
# subnormals below 2^-6, 448 the largest; S.1111.111 is NaN), as a sorted table of
# (value, code) used to round float32 data to the nearest E4M3 code.
_E4M3_CODES = np.array([c for c in range(0x7F)], dtype=np.uint8)
_E4M3_VALUES = np.array([((c & 7) / 8.0) * 2.0 ** -6 if (c >> 3) == 0 else (1 + (c & 7) / 8.0) * 2.0 ** ((c >> 3) - 7)
                         for c in range(0x7F)], dtype=np.float64)
E4M3_NAN = np.uint8(0x7F)


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round to the nearest OCP E4M3 code (ties to an even code), saturating at +-448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    hi = np.clip(np.searchsorted(_E4M3_VALUES, a), 1, len(_E4M3_VALUES) - 1)
    lo = hi - 1
    dlo, dhi = a - _E4M3_VALUES[lo], _E4M3_VALUES[hi] - a
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(_E4M3_CODES[lo] % 2 == 0, lo, hi)))
    code = _E4M3_CODES[pick]
    return np.where(x < 0, code | np.uint8(0x80), code).astype(np.uint8)


def _normal(rng, shape, dtype):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return f32_to_bf16_bits(x) if dtype == BF16 else x


def cache_capacity(max_prefix: int, D: int) -> int:
    """Room for the longest prefix plus one appended block, rounded up to 64 slots."""
    return ((max_prefix + D + 63) // 64) * 64


def params_for(cfg_id: int, **overrides) -> dict:
    p = dict(CONFIGS[cfg_id])
    p.update(overrides)
    return p


def make_step(p: dict, seed: int, plant_L=None) -> dict:
    """Draw one step's inputs for parameter dict ``p`` (a config, possibly overridden).

    ``plant_L`` forces the accepted-prefix length of a speculative plant
    (used for the L = 0 and L = D edge cases).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    n, D, Hq, Hkv, d = p["n_items"], p["D"], p["Hq"], p["Hkv"], p["d"]
    dtype = p["dtype"]
    kind = p["prefix"][0]
    if kind == "fixed":
        prefix = np.full(n, p["prefix"][1], dtype=np.int32)
    elif kind == "uniform":
        lo, hi = p["prefix"][1], p["prefix"][2]
        prefix = rng.integers(lo, hi + 1, size=n, dtype=np.int64).astype(np.int32)
    elif kind == "list":
        prefix = np.asarray(p["prefix"][1], dtype=np.int32)
        assert prefix.shape == (n,)
    else:
        raise ValueError(kind)
    max_prefix = int(prefix.max()) if n else 0
    cap = p.get("cap") or cache_capacity(max_prefix, D)
    if dtype == FP8KV:
        return _make_step_fp8kv(p, rng, prefix, cap, plant_L, seed)
    elem = np.uint16 if dtype == BF16 else np.float32
    nan = BF16_NAN if dtype == BF16 else np.float32(np.nan)

    q = _normal(rng, (n, D, Hq, d), dtype)
    k_cache = np.full((n, Hkv, cap, d), nan, dtype=elem)
    v_cache = np.full((n, Hkv, cap, d), nan, dtype=elem)
    for it in range(n):
        P = int(prefix[it])
        k_cache[it, :, :P, :] = _normal(rng, (Hkv, P, d), dtype)
    for it in range(n):
        P = int(prefix[it])
        v_cache[it, :, :P, :] = _normal(rng, (Hkv, P, d), dtype)
    k_blk = _normal(rng, (n, D, Hkv, d), dtype)
    v_blk = _normal(rng, (n, D, Hkv, d), dtype)

    n_req, V = p["n_req"], p["V"]
    masked = np.zeros((n_req, D), dtype=np.uint8)
    tokens = np.full((n_req, D), -1, dtype=np.int32)
    for r in range(n_req):
        perm = rng.permutation(D)
        masked[r, perm[: p["n_masked"]]] = 1
    for r in range(n_req):
        ids = rng.integers(0, V, size=D, dtype=np.int64).astype(np.int32)
        tokens[r] = np.where(masked[r] == 1, -1, ids)

    std = np.float32(np.sqrt(p["logit_sigma2"]))
    logits = rng.standard_normal(size=(n_req, D, V), dtype=np.float32) * std

    out = dict(params=p, seed=seed, cap=cap, prefix=prefix, q=q, k_cache=k_cache,
               v_cache=v_cache, k_blk=k_blk, v_blk=v_blk, masked=masked, tokens=tokens,
               logits=logits)

    plant = p.get("plant")
    if plant == "peak8":
        for r in range(n_req):
            for i in range(D):
                v_star = int(rng.integers(0, V))
                logits[r, i, v_star] = logits[r, i].max() + np.float32(8.0)
    elif plant == "geom0.3":
        draft = rng.integers(0, V, size=(n_req, D), dtype=np.int64).astype(np.int32)
        Ls = np.zeros(n_req, dtype=np.int32)
        for r in range(n_req):
            L = int(rng.geometric(0.3)) - 1  # P(L = l) = 0.3 * 0.7**l, l >= 0
            if plant_L is not None:
                L = int(plant_L)
            L = min(L, D)
            Ls[r] = L
            for i in range(L):
                logits[r, i, draft[r, i]] = logits[r, i].max() + np.float32(8.0)
            if L < D:
                logits[r, L, draft[r, L]] = logits[r, L].min() - np.float32(1.0)
        out["draft"] = draft
        out["planted_L"] = Ls
    return out


def fresh_logits(p: dict, rng: np.random.Generator) -> np.ndarray:
    """Logits for a later denoising step of the same block (no plant)."""
    std = np.float32(np.sqrt(p["logit_sigma2"]))
    return rng.standard_normal(size=(p["n_req"], p["D"], p["V"]), dtype=np.float32) * std


def config_step(cfg_id: int, **overrides) -> dict:
    """The canonical seeded step of a config (seed 1000 + config number)."""
    return make_step(params_for(cfg_id, **overrides), seed_of(cfg_id))


def make_lmhead(p: dict, seed: int) -> dict:
    """Draw the inputs of one LM-head + confidence step.

    Layouts: hidden bf16 [n_req][D][H], weight bf16 [V][H] (a linear layer's
    row-major weight), masked u8 [n_req][D], tokens i32 [n_req][D].
    Draw order: hidden, weight, masked set, committed ids, planted tokens.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    n_req, D, V, H = p["n_req"], p["D"], p["V"], p["H"]
    hidden = f32_to_bf16_bits(rng.standard_normal(size=(n_req, D, H), dtype=np.float32))
    w_std = np.float32(2.0 / np.sqrt(H))
    weight = np.empty((V, H), dtype=np.uint16)
    step = 1 << 14
    for v0 in range(0, V, step):  # in slices, to bound the float32 temporary
        v1 = min(V, v0 + step)
        weight[v0:v1] = f32_to_bf16_bits(rng.standard_normal(size=(v1 - v0, H), dtype=np.float32) * w_std)
    masked = np.zeros((n_req, D), dtype=np.uint8)
    tokens = np.full((n_req, D), -1, dtype=np.int32)
    for r in range(n_req):
        masked[r, rng.permutation(D)[: p["n_masked"]]] = 1
    for r in range(n_req):
        ids = rng.integers(0, V, size=D, dtype=np.int64).astype(np.int32)
        tokens[r] = np.where(masked[r] == 1, -1, ids)
    planted = []
    scale = np.float32(p["gain"] / H)
    for r in range(n_req):
        rows = np.flatnonzero(masked[r])[: p["plants"]]
        for i in rows:
            v_star = int(rng.integers(0, V))
            weight[v_star] = f32_to_bf16_bits(bf16_bits_to_f32(hidden[r, i]) * scale)
            planted.append((r, int(i), v_star))
    return dict(params=p, seed=seed, hidden=hidden, weight=weight, masked=masked, tokens=tokens,
                planted=planted)


def lmhead_step(cfg_id: int, **overrides) -> dict:
    p = dict(LMHEAD_CONFIGS[cfg_id])
    p.update(overrides)
    return make_lmhead(p, lmhead_seed_of(cfg_id))


def _make_step_fp8kv(p, rng, prefix, cap, plant_L, seed):
    """The FP8-KV variant of make_step: queries bf16; the cache and block keys and
    values drawn as float32 N(0, 1) in make_step's order, then stored as OCP E4M3
    codes of value / scale, one fp32 scale per (item, KV head): the largest
    magnitude over that head's valid cache entries and block entries, over 448.
    Cache slots past the prefix hold the E4M3 NaN code.  Logits, masked set and
    plants follow make_step (a bf16-dtype draw of the same parameters)."""
    n, D, Hq, Hkv, d = p["n_items"], p["D"], p["Hq"], p["Hkv"], p["d"]
    q = _normal(rng, (n, D, Hq, d), BF16)
    kf = [rng.standard_normal(size=(Hkv, int(prefix[it]), d), dtype=np.float32) for it in range(n)]
    vf = [rng.standard_normal(size=(Hkv, int(prefix[it]), d), dtype=np.float32) for it in range(n)]
    kbf = rng.standard_normal(size=(n, D, Hkv, d), dtype=np.float32)
    vbf = rng.standard_normal(size=(n, D, Hkv, d), dtype=np.float32)
    k_scale = np.zeros((n, Hkv), np.float32)
    v_scale = np.zeros((n, Hkv), np.float32)
    for it in range(n):
        for g in range(Hkv):
            k_scale[it, g] = max(float(np.abs(kf[it][g]).max(initial=0.0)), float(np.abs(kbf[it, :, g]).max())) / 448.0
            v_scale[it, g] = max(float(np.abs(vf[it][g]).max(initial=0.0)), float(np.abs(vbf[it, :, g]).max())) / 448.0
    k_cache = np.full((n, Hkv, cap, d), E4M3_NAN, dtype=np.uint8)
    v_cache = np.full((n, Hkv, cap, d), E4M3_NAN, dtype=np.uint8)
    k_blk = np.zeros((n, D, Hkv, d), np.uint8)
    v_blk = np.zeros((n, D, Hkv, d), np.uint8)
    for it in range(n):
        P = int(prefix[it])
        for g in range(Hkv):
            k_cache[it, g, :P, :] = f32_to_e4m3_bits(kf[it][g] / k_scale[it, g])
            v_cache[it, g, :P, :] = f32_to_e4m3_bits(vf[it][g] / v_scale[it, g])
            k_blk[it, :, g, :] = f32_to_e4m3_bits(kbf[it, :, g] / k_scale[it, g])
            v_blk[it, :, g, :] = f32_to_e4m3_bits(vbf[it, :, g] / v_scale[it, g])
    rest = make_step(dict(p, dtype=BF16, n_items=1, prefix=("fixed", 0), Hq=1, Hkv=1, d=8), seed + 7919)
    return dict(params=p, seed=seed, cap=cap, prefix=prefix, q=q, k_cache=k_cache, v_cache=v_cache,
                k_blk=k_blk, v_blk=v_blk, k_scale=k_scale, v_scale=v_scale, masked=rest["masked"],
                tokens=rest["tokens"], logits=rest["logits"], **{k: rest[k] for k in ("draft", "planted_L") if k in rest})


def quad_slot_count(B: int) -> int:
    """Block slots of a quadratic self-speculative step (layout only): B drafts,
    then B - g mask tokens for each group g = 0..B-1."""
    return B * (B + 3) // 2


def make_quad_step(p: dict, seed: int) -> dict:
    """Inputs of one quadratic self-speculative attention step: make_step's draws
    (prefix, Q, cache K/V, block K/V) with quad_slot_count(B) block slots.  The
    commit-side fields are drawn for one request over 2 tokens and are unused.
    ``params`` keeps D = slot count, B and mode = QUAD."""
    B = int(p["B"])
    S = quad_slot_count(B)
    q = dict(p, D=S, mode=QUAD, n_req=1, n_masked=0, V=2, plant=None, S=1, tau=1.0, logit_sigma2=1.0)
    st = make_step(q, seed)
    st["params"] = q
    return st


def quad_step(cfg_id: int, **overrides) -> dict:
    """The canonical seeded quadratic step (seed 3000 + config number)."""
    p = dict(QUAD_CONFIGS[cfg_id])
    p.update(overrides)
    return make_quad_step(p, quad_seed_of(cfg_id))


def make_two_stream(p: dict, seed: int) -> dict:
    """Inputs of one two-stream training attention call.

    Sequence layout: clean stream = vision, then each turn's prompt and response;
    noisy stream = the responses' tokens in order (padding after them when a
    sequence has fewer response tokens than the longest).  Lc and Ln are the
    maxima over sequences; a shorter clean stream ends in plain clean tokens.
    Arrays: q [n][L][Hq][d] with L = Lc + Ln; k and v [n][Hkv][cap][d]
    (cap = L rounded up to p["cap_align"], default 64, zeros past L); spans int32
    [n][max_spans][2] = (clean start, length) of each response; n_spans [n].
    Draw order: q, then k, then v, as N(0, 1) rounded to bf16.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    n, Hq, Hkv, d, dtype = p["n_seq"], p["Hq"], p["Hkv"], p["d"], p["dtype"]
    turns = p["turns"]
    per_seq = turns if isinstance(turns[0], list) else [turns] * n
    assert len(per_seq) == n
    spans_l, lc_l, ln_l = [], [], []
    for t in per_seq:
        pos, sp = p["vision"], []
        for prompt, resp in t:
            pos += prompt
            sp.append((pos, resp))
            pos += resp
        spans_l.append(sp)
        lc_l.append(pos)
        ln_l.append(sum(r for _, r in sp))
    Lc, Ln = max(lc_l), max(ln_l)
    L = Lc + Ln
    align = int(p.get("cap_align", 64))
    cap = (L + align - 1) // align * align
    max_spans = max(len(sp) for sp in spans_l)
    spans = np.zeros((n, max_spans, 2), np.int32)
    n_spans = np.zeros(n, np.int32)
    for i, sp in enumerate(spans_l):
        n_spans[i] = len(sp)
        for r, (c, ln) in enumerate(sp):
            spans[i, r] = (c, ln)
    elem = np.uint16 if dtype == BF16 else np.float32
    q = _normal(rng, (n, L, Hq, d), dtype)
    k = np.zeros((n, Hkv, cap, d), elem)
    v = np.zeros((n, Hkv, cap, d), elem)
    k[:, :, :L, :] = _normal(rng, (n, Hkv, L, d), dtype)
    v[:, :, :L, :] = _normal(rng, (n, Hkv, L, d), dtype)
    return dict(params=dict(p, Lc=Lc, Ln=Ln, L=L), seed=seed, q=q, k=k, v=v, spans=spans, n_spans=n_spans,
                cap=cap, Lc=Lc, Ln=Ln)


def two_stream_step(cfg_id: int, **overrides) -> dict:
    p = dict(TWO_STREAM_CONFIGS[cfg_id])
    p.update(overrides)
    return make_two_stream(p, two_stream_seed_of(cfg_id))
