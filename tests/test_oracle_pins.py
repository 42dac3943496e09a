"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test checks the oracle against something it does not share code with:
a dense attention mask built from the pages' three mask rules and evaluated
by torch's SDPA in float64, library routines (scipy ``logsumexp``, numpy
``argmax``), closed forms, brute force over all choices on tiny inputs,
invariants, and the worked example printed on the pages
(``tests/golden/commit_k.json``).
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth
from synth import BF16, BIDIR, CAUSAL, F32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _widen(a):
    return synth.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def _rand(rng, shape, dtype):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return synth.f32_to_bf16_bits(x) if dtype == BF16 else x


def _pack_cache(k_seq, v_seq, cap, dtype):
    """k_seq/v_seq: [Hkv][P][d] -> cache layout [1][Hkv][cap][d] (NaN tail)."""
    Hkv, P, d = k_seq.shape
    el = np.uint16 if dtype == BF16 else np.float32
    nan = synth.gen.BF16_NAN if dtype == BF16 else np.float32(np.nan)
    kc = np.full((1, Hkv, cap, d), nan, el)
    vc = np.full((1, Hkv, cap, d), nan, el)
    kc[0, :, :P, :] = k_seq
    vc[0, :, :P, :] = v_seq
    return kc, vc


def _sdpa(q, k, v, mask, group):
    """torch SDPA in float64; q [Hq][Lq][d], k/v [Hkv][Lk][d], mask [Lq][Lk] bool."""
    qt = torch.from_numpy(q)[None]
    kt = torch.from_numpy(k).repeat_interleave(group, dim=0)[None]
    vt = torch.from_numpy(v).repeat_interleave(group, dim=0)[None]
    m = None if mask is None else torch.from_numpy(mask)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m)[0].numpy()


# ---------------------------------------------------------------------------
# Attention: two-stream training mask (Fast-dVLM write-up section 4.1; summary
# page Fig. 3) evaluated densely, versus the oracle's per-block inference form.
# ---------------------------------------------------------------------------

def _two_stream_mask(n_vis, n_txt, D, B):
    """Mask over [noisy stream w ; clean stream x] built from the three rules:
    M_N2N block-diagonal among noisy tokens; M_N2C noisy block b sees vision,
    prompt text and clean blocks before b; M_C2C clean tokens causal.  Clean
    tokens never see noisy ones.  Vision lives only in the clean stream."""
    Ln = B * D
    Lp = n_vis + n_txt
    Lc = Lp + B * D
    L = Ln + Lc
    mask = np.zeros((L, L), dtype=bool)
    for b in range(B):
        rows = slice(b * D, (b + 1) * D)
        mask[rows, b * D:(b + 1) * D] = True                # M_N2N
        mask[rows, Ln:Ln + Lp] = True                        # M_N2C: vision + prompt
        mask[rows, Ln + Lp:Ln + Lp + b * D] = True           # M_N2C: earlier clean blocks
    for c in range(Lc):
        mask[Ln + c, Ln:Ln + c + 1] = True                   # M_C2C
    return mask


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("Hq,Hkv,d", [(2, 1, 8), (4, 2, 16), (6, 3, 8)])
def test_attention_matches_two_stream_dense_mask(dtype, Hq, Hkv, d):
    rng = np.random.Generator(np.random.PCG64(7 + Hq + d))
    n_vis, n_txt, D, B = 5, 3, 4, 3
    Ln, Lp = B * D, n_vis + n_txt
    Lc = Lp + B * D
    L = Ln + Lc
    group = Hq // Hkv
    Q = _rand(rng, (Hq, L, d), dtype)
    K = _rand(rng, (Hkv, L, d), dtype)
    V = _rand(rng, (Hkv, L, d), dtype)
    ref = _sdpa(_widen(Q), _widen(K), _widen(V), _two_stream_mask(n_vis, n_txt, D, B), group)
    for b in range(B):
        P = Lp + b * D
        cap = P + D + 3
        ctx = slice(Ln, Ln + P)                               # clean positions before block b
        kc, vc = _pack_cache(K[:, ctx], V[:, ctx], cap, dtype)
        # Noisy block b: denoise attention (bidirectional inside the block).
        nz = slice(b * D, (b + 1) * D)
        q = np.ascontiguousarray(np.swapaxes(Q[:, nz], 0, 1))[None]
        kb = np.ascontiguousarray(np.swapaxes(K[:, nz], 0, 1))[None]
        vb = np.ascontiguousarray(np.swapaxes(V[:, nz], 0, 1))[None]
        out = oracle.attention(q, kb, vb, kc, vc, np.array([P], np.int32), BIDIR)
        np.testing.assert_allclose(out[0], np.swapaxes(ref[:, nz], 0, 1), rtol=0, atol=1e-12)
        # Clean block b: the causal (verify / AR) pass over the filled block.
        cl = slice(Ln + P, Ln + P + D)
        q = np.ascontiguousarray(np.swapaxes(Q[:, cl], 0, 1))[None]
        kb = np.ascontiguousarray(np.swapaxes(K[:, cl], 0, 1))[None]
        vb = np.ascontiguousarray(np.swapaxes(V[:, cl], 0, 1))[None]
        out = oracle.attention(q, kb, vb, kc, vc, np.array([P], np.int32), CAUSAL)
        np.testing.assert_allclose(out[0], np.swapaxes(ref[:, cl], 0, 1), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Quadratic self-speculative attention (Fast-dVLM write-up, section 5.3, the
# quadratic variant): the oracle's compact slot form against (a) the causal
# verify pass over the drafts, (b) a denoise pass per acceptance hypothesis,
# and (c) the literal B x B expansion evaluated with a dense mask by SDPA.
# ---------------------------------------------------------------------------

def _quad_layout(B):
    """[(group, token)] of the compact slots: drafts (-1, t), then (g, t) for t = g..B-1."""
    return [(-1, t) for t in range(B)] + [(g, t) for g in range(B) for t in range(g, B)]


def _quad_inputs(rng, B, Hq, Hkv, d, P, dtype):
    S = oracle.quad_slots(B)
    q = _rand(rng, (1, S, Hq, d), dtype)
    kb = _rand(rng, (1, S, Hkv, d), dtype)
    vb = _rand(rng, (1, S, Hkv, d), dtype)
    kseq = _rand(rng, (Hkv, P, d), dtype)
    vseq = _rand(rng, (Hkv, P, d), dtype)
    return q, kb, vb, kseq, vseq


@pytest.mark.parametrize("B", [1, 2, 5])
def test_quad_draft_rows_are_the_causal_verify_pass(B):
    rng = np.random.Generator(np.random.PCG64(60 + B))
    Hq, Hkv, d, P = 4, 2, 8, 9
    q, kb, vb, kseq, vseq = _quad_inputs(rng, B, Hq, Hkv, d, P, F32)
    kc, vc = _pack_cache(kseq, vseq, P + oracle.quad_slots(B) + 2, F32)
    pre = np.array([P], np.int32)
    out = oracle.attention_quad(q, kb, vb, kc, vc, pre, B)
    ref = oracle.attention(q[:, :B], kb[:, :B], vb[:, :B], kc, vc, pre, CAUSAL)
    np.testing.assert_allclose(out[:, :B], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("B", [1, 3, 6])
def test_quad_group_rows_are_a_denoise_pass_over_the_accepted_drafts(B):
    """Group g's mask tokens see the cache plus drafts 0..g-1 as context and their
    own group bidirectionally: a denoise step whose cache holds those drafts."""
    rng = np.random.Generator(np.random.PCG64(70 + B))
    Hq, Hkv, d, P = 6, 3, 8, 7
    q, kb, vb, kseq, vseq = _quad_inputs(rng, B, Hq, Hkv, d, P, BF16)
    cap = P + oracle.quad_slots(B) + 4
    kc, vc = _pack_cache(kseq, vseq, cap, BF16)
    out = oracle.attention_quad(q, kb, vb, kc, vc, np.array([P], np.int32), B)
    slots = _quad_layout(B)
    for g in range(B):
        rows = [i for i, (gg, _) in enumerate(slots) if gg == g]
        ctx_k = np.concatenate([kseq, np.swapaxes(kb[0, :g], 0, 1)], axis=1)
        ctx_v = np.concatenate([vseq, np.swapaxes(vb[0, :g], 0, 1)], axis=1)
        kc_g, vc_g = _pack_cache(ctx_k, ctx_v, cap, BF16)
        ref = oracle.attention(q[:, rows], kb[:, rows], vb[:, rows], kc_g, vc_g, np.array([P + g], np.int32), BIDIR)
        np.testing.assert_allclose(out[:, rows], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("B", [2, 4])
def test_quad_matches_the_b_by_b_expansion_with_a_dense_mask(B):
    """The literal form: B groups of B tokens, group g = drafts 0..g-1 then B - g mask
    tokens; inside a group drafts are causal and mask tokens see the whole group; no
    group sees another; all see the cache.  Evaluated densely by SDPA over
    [cache ; B*B expanded tokens]; every expanded row equals its compact slot's row."""
    rng = np.random.Generator(np.random.PCG64(80 + B))
    Hq, Hkv, d, P = 4, 1, 16, 11
    q, kb, vb, kseq, vseq = _quad_inputs(rng, B, Hq, Hkv, d, P, F32)
    kc, vc = _pack_cache(kseq, vseq, P + oracle.quad_slots(B), F32)
    out = oracle.attention_quad(q, kb, vb, kc, vc, np.array([P], np.int32), B)
    slots = _quad_layout(B)
    index = {gt: i for i, gt in enumerate(slots)}
    src = []                                   # compact slot of every expanded token
    for g in range(B):
        src += [index[(-1, t)] for t in range(g)] + [index[(g, t)] for t in range(g, B)]
    L = B * B
    mask = np.zeros((L, P + L), bool)
    mask[:, :P] = True
    for g in range(B):
        for t in range(B):
            for t2 in range(B):
                mask[g * B + t, P + g * B + t2] = (t >= g) or (t2 <= t)
    Q = np.swapaxes(q[0, src], 0, 1)
    K = np.concatenate([kseq, np.swapaxes(kb[0, src], 0, 1)], axis=1)
    V = np.concatenate([vseq, np.swapaxes(vb[0, src], 0, 1)], axis=1)
    ref = _sdpa(_widen(Q), _widen(K), _widen(V), mask, Hq // Hkv)
    np.testing.assert_allclose(out[0, src], np.swapaxes(ref, 0, 1), rtol=0, atol=1e-12)


def _random_step(rng, n, D, Hq, Hkv, d, P, dtype, cap=None):
    prefix = np.asarray(P, np.int32)
    cap = cap or int(prefix.max()) + D + 5
    q = _rand(rng, (n, D, Hq, d), dtype)
    kb = _rand(rng, (n, D, Hkv, d), dtype)
    vb = _rand(rng, (n, D, Hkv, d), dtype)
    el = np.uint16 if dtype == BF16 else np.float32
    nan = synth.gen.BF16_NAN if dtype == BF16 else np.float32(np.nan)
    kc = np.full((n, Hkv, cap, d), nan, el)
    vc = np.full((n, Hkv, cap, d), nan, el)
    for it in range(n):
        p = int(prefix[it])
        kc[it, :, :p] = _rand(rng, (Hkv, p, d), dtype)
        vc[it, :, :p] = _rand(rng, (Hkv, p, d), dtype)
    return q, kb, vb, kc, vc, prefix


def _keys_natural(kc, vc, kb, vb, it, P):
    """Key/value sequences [Hkv][P+D][d] of item ``it`` in natural layout."""
    k = np.concatenate([kc[it, :, :P], np.swapaxes(kb[it], 0, 1)], axis=1)
    v = np.concatenate([vc[it, :, :P], np.swapaxes(vb[it], 0, 1)], axis=1)
    return k, v


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_single_slot_is_textbook_decode(dtype):
    """D = 1: the block step is ordinary single-query decode over P + 1 keys
    (each block opens with one AR step: Fast-dVLM write-up, section 5.1)."""
    rng = np.random.Generator(np.random.PCG64(11))
    n, Hq, Hkv, d = 3, 4, 2, 16
    q, kb, vb, kc, vc, prefix = _random_step(rng, n, 1, Hq, Hkv, d, [0, 9, 40], dtype)
    o_c = oracle.attention(q, kb, vb, kc, vc, prefix, CAUSAL)
    o_b = oracle.attention(q, kb, vb, kc, vc, prefix, BIDIR)
    np.testing.assert_array_equal(o_c, o_b)
    for it in range(n):
        k, v = _keys_natural(kc, vc, kb, vb, it, int(prefix[it]))
        ref = _sdpa(np.swapaxes(_widen(q[it]), 0, 1), _widen(k), _widen(v), None, Hq // Hkv)
        np.testing.assert_allclose(o_c[it], np.swapaxes(ref, 0, 1), rtol=0, atol=1e-12)


def test_empty_prefix_bidir_is_full_attention_over_block():
    rng = np.random.Generator(np.random.PCG64(12))
    q, kb, vb, kc, vc, prefix = _random_step(rng, 1, 6, 4, 1, 8, [0], F32)
    out = oracle.attention(q, kb, vb, kc, vc, prefix, BIDIR)
    ref = _sdpa(np.swapaxes(_widen(q[0]), 0, 1), _widen(np.swapaxes(kb[0], 0, 1)),
                _widen(np.swapaxes(vb[0], 0, 1)), None, 4)
    np.testing.assert_allclose(out[0], np.swapaxes(ref, 0, 1), rtol=0, atol=1e-12)


def test_causal_with_cache_is_chunked_prefill():
    """CAUSAL with a cache equals causal attention over the concatenated sequence (rows of the block)."""
    rng = np.random.Generator(np.random.PCG64(13))
    D, P = 5, 17
    q, kb, vb, kc, vc, prefix = _random_step(rng, 1, D, 2, 2, 8, [P], F32)
    out = oracle.attention(q, kb, vb, kc, vc, prefix, CAUSAL)
    k, v = _keys_natural(kc, vc, kb, vb, 0, P)
    mask = np.tril(np.ones((P + D, P + D), bool))[P:]
    ref = _sdpa(np.swapaxes(_widen(q[0]), 0, 1), _widen(k), _widen(v), mask, 1)
    np.testing.assert_allclose(out[0], np.swapaxes(ref, 0, 1), rtol=0, atol=1e-12)


def test_attention_invariants():
    rng = np.random.Generator(np.random.PCG64(14))
    n, D, Hq, Hkv, d = 2, 4, 4, 2, 8
    q, kb, vb, kc, vc, prefix = _random_step(rng, n, D, Hq, Hkv, d, [20, 33], F32)
    base = oracle.attention(q, kb, vb, kc, vc, prefix, BIDIR)
    assert np.all(np.isfinite(base)), "NaN canaries past the prefix must never be read"
    # Constant values give that constant, whatever the scores.
    vc2, vb2 = vc.copy(), vb.copy()
    for it in range(n):
        vc2[it, :, :prefix[it]] = 0.75
    vb2[:] = 0.75
    const = oracle.attention(q, kb, vb2, kc, vc2, prefix, BIDIR)
    np.testing.assert_allclose(const, 0.75, rtol=0, atol=1e-14)
    # Permuting prefix positions (keys with their values) changes nothing.
    kc3, vc3 = kc.copy(), vc.copy()
    for it in range(n):
        P = int(prefix[it])
        perm = rng.permutation(P)
        kc3[it, :, :P] = kc[it, :, perm].swapaxes(0, 1)
        vc3[it, :, :P] = vc[it, :, perm].swapaxes(0, 1)
    perm_out = oracle.attention(q, kb, vb, kc3, vc3, prefix, BIDIR)
    np.testing.assert_allclose(perm_out, base, rtol=0, atol=1e-12)
    # CAUSAL differs from BIDIR only in the block: the last slot sees the whole block either way.
    caus = oracle.attention(q, kb, vb, kc, vc, prefix, CAUSAL)
    np.testing.assert_allclose(caus[:, D - 1], base[:, D - 1], rtol=0, atol=1e-13)
    assert not np.allclose(caus[:, 0], base[:, 0])


def test_gqa_grouping_is_contiguous():
    """Heads 0..G-1 share KV head 0 (contiguous grouping): with identical queries per
    group, every head of a group must give the same output and the groups differ."""
    rng = np.random.Generator(np.random.PCG64(15))
    q, kb, vb, kc, vc, prefix = _random_step(rng, 1, 3, 6, 2, 8, [10], F32)
    q[:, :, :, :] = q[:, :, :1, :]
    out = oracle.attention(q, kb, vb, kc, vc, prefix, BIDIR)
    np.testing.assert_array_equal(out[:, :, 1], out[:, :, 0])
    np.testing.assert_array_equal(out[:, :, 2], out[:, :, 0])
    np.testing.assert_array_equal(out[:, :, 4], out[:, :, 3])
    assert not np.allclose(out[:, :, 3], out[:, :, 0])


# ---------------------------------------------------------------------------
# Confidence (DiffusionVL notes, cached block decoding: confidence is the
# probability of the chosen token).
# ---------------------------------------------------------------------------

def test_confidence_matches_logsumexp_and_argmax():
    rng = np.random.Generator(np.random.PCG64(21))
    for V, sig in [(2, 1.0), (1000, math.sqrt(3)), (151936, 2.0)]:
        x = (rng.standard_normal(V, dtype=np.float32) * np.float32(sig))
        conf, a, lse, p2 = oracle.confidence_row(x)
        assert a == int(np.argmax(x))
        ref_lse = scipy.special.logsumexp(x.astype(np.float64))
        assert abs(lse - ref_lse) <= 1e-12 * max(1.0, abs(ref_lse))
        assert abs(conf - math.exp(float(x[a]) - ref_lse)) <= 1e-14
        xs = np.sort(x.astype(np.float64))
        assert abs(p2 - math.exp(xs[-2] - ref_lse)) <= 1e-14


def test_confidence_closed_forms():
    V = 50
    conf, a, _, _ = oracle.confidence_row(np.full(V, 0.3, np.float32))
    assert a == 0 and abs(conf - 1.0 / V) < 1e-15
    x = np.full(V, -1.0, np.float32)
    x[17] = 2.0
    conf, a, _, _ = oracle.confidence_row(x)
    ref = math.exp(2.0) / (math.exp(2.0) + (V - 1) * math.exp(-1.0))
    assert a == 17 and abs(conf - ref) < 1e-15
    # Shift invariance (integer logits keep the shift exact in fp32).
    rng = np.random.Generator(np.random.PCG64(22))
    xi = rng.integers(-20, 20, size=300).astype(np.float32)
    c0, a0, _, _ = oracle.confidence_row(xi)
    c1, a1, _, _ = oracle.confidence_row(xi + np.float32(64.0))
    assert a0 == a1 and abs(c0 - c1) < 1e-15
    # Ties go to the lowest index.
    x = np.zeros(10, np.float32)
    x[[7, 3, 9]] = 5.0
    assert oracle.confidence_row(x)[1] == 3


# ---------------------------------------------------------------------------
# Commit rule (DiffusionVL notes, Algorithm 1 and the dynamic rule).
# ---------------------------------------------------------------------------

def test_commit_k_matches_pages_worked_example():
    with open(os.path.join(GOLDEN, "commit_k.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        assert oracle.commit_k(c["D"], c["S"], c["n_masked"]) == c["k"], c


def _brute_commit(conf, masked, k, tau):
    """Top-k by exhaustive search: the unique k-subset of M whose every member
    outranks every non-member under (confidence desc, index asc); plus {c > tau}."""
    M = [i for i in range(len(masked)) if masked[i]]
    before = lambda a, b: conf[a] > conf[b] or (conf[a] == conf[b] and a < b)
    tops = [set(T) for T in itertools.combinations(M, k)
            if all(before(t, u) for t in T for u in M if u not in T)]
    assert len(tops) == 1
    return tops[0] | {i for i in M if conf[i] > tau}


def _logits_for_conf(rng, D, V):
    return (rng.standard_normal((1, D, V), dtype=np.float32) * np.float32(1.5))


@pytest.mark.parametrize("D", [1, 2, 3, 4, 5, 6])
def test_commit_brute_force_small_blocks(D):
    rng = np.random.Generator(np.random.PCG64(30 + D))
    V = 7
    for trial in range(60):
        logits = _logits_for_conf(rng, D, V)
        if trial % 5 == 0:                       # force exact confidence ties
            logits[0, :] = logits[0, 0]
        masked = rng.integers(0, 2, size=(1, D)).astype(np.uint8)
        tokens = np.where(masked == 1, -1, 5).astype(np.int32)
        S = int(rng.integers(1, D + 2))
        tau = float(rng.choice([0.2, 0.35, 0.5, 0.9, 1.0]))
        r = oracle.confidence_commit(logits, masked, tokens, S, tau)
        conf = r["conf"][0]
        # The rule is decided on the fp64 confidences; check them against
        # their definition first (the probability of the greedy token).
        for i in np.flatnonzero(masked[0]):
            x = logits[0, i].astype(np.float64)
            assert abs(conf[i] - 1.0 / np.exp(x - x.max()).sum()) < 1e-15
        k = min(-(-D // S), int(masked.sum()))
        want = _brute_commit(conf, masked[0], k, tau)
        got = set(np.nonzero(r["committed"][0])[0].tolist())
        assert got == want, (trial, conf, masked, k, tau)
        for i in range(D):
            if masked[0, i]:
                assert r["argmax"][0, i] == int(np.argmax(logits[0, i]))
            else:
                assert r["tokens"][0, i] == tokens[0, i] and np.isnan(r["conf"][0, i])


def test_commit_threshold_is_strict():
    """'greater than tau': a confidence exactly equal to tau is not taken by the threshold."""
    D, V = 4, 2
    logits = np.zeros((1, D, V), np.float32)       # rows 1..3: conf exactly 0.5
    logits[0, 0] = [10.0, 0.0]                     # row 0 wins the single top-k slot
    masked = np.ones((1, D), np.uint8)
    tokens = np.full((1, D), -1, np.int32)
    r = oracle.confidence_commit(logits, masked, tokens, S=4, tau=0.5)
    assert r["committed"][0].tolist() == [1, 0, 0, 0]
    r = oracle.confidence_commit(logits, masked, tokens, S=4, tau=0.4999)
    assert r["committed"][0].tolist() == [1, 1, 1, 1]


def _run_block(p, seed, logits0, masked, tokens):
    """Multi-step denoising of one block with fresh logits per step."""
    rng = np.random.Generator(np.random.PCG64(seed))
    steps, history = 0, []
    logits = logits0
    while masked.sum() > 0:
        before_tokens = tokens.copy()
        before_masked = masked.copy()
        r = oracle.confidence_commit(logits, masked, tokens, p["S"], p["tau"])
        masked, tokens = r["masked"], r["tokens"]
        steps += 1
        history.append((before_masked, before_tokens, r))
        logits = synth.fresh_logits(p, rng)
        assert steps <= p["S"] + 1
    return steps, history


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_multistep_invariants(cfg):
    """Committed tokens stay fixed; each step commits at least min(k, |M|);
    a block finishes within S steps (DiffusionVL notes, cached block decoding)."""
    s = synth.config_step(cfg)
    p = s["params"]
    steps, hist = _run_block(p, 99, s["logits"], s["masked"].copy(), s["tokens"].copy())
    assert steps <= p["S"]
    for before_m, before_t, r in hist:
        for rq in range(p["n_req"]):
            nm = int(before_m[rq].sum())
            k = oracle.commit_k(p["D"], p["S"], nm)
            assert int(r["n_committed"][rq]) >= k
            keep = before_m[rq] == 0
            np.testing.assert_array_equal(r["tokens"][rq][keep], before_t[rq][keep])
            assert np.all(r["masked"][rq][keep] == 0)
    if cfg == 2:
        # Planted +8 peaks put most confidences near 0.93-0.98 (> tau = 0.9): most of
        # the block commits in the first step through the threshold rule.
        first = hist[0][2]
        assert int(first["n_committed"][0]) >= 6 and steps <= 2
        c = first["conf"][0]
        for i in range(p["D"]):
            if first["committed"][0, i] and c[i] <= p["tau"]:
                assert c[i] == np.nanmax(c)


def test_threshold_off_gives_closed_form_step_count():
    """With tau >= 1 nothing passes the threshold: exactly ceil(|M0| / ceil(D/S)) steps."""
    for (D, S, nm) in [(8, 8, 8), (8, 4, 8), (16, 16, 8), (32, 8, 32), (16, 5, 11)]:
        p = synth.params_for(1, D=D, S=S, n_masked=nm, tau=1.0, V=64)
        s = synth.make_step(p, seed=5)
        steps, _ = _run_block(p, 6, s["logits"], s["masked"].copy(), s["tokens"].copy())
        k = -(-D // S)
        assert steps == -(-nm // k), (D, S, nm, steps)


# ---------------------------------------------------------------------------
# Speculative verify and KV append (Fast-dVLM write-up, section 5.3).
# ---------------------------------------------------------------------------

def test_verify_recovers_planted_prefix():
    for seed in range(40):
        s = synth.make_step(synth.params_for(4, V=3000, prefix=("fixed", 8)), seed)
        L, amax = oracle.spec_verify(s["logits"], s["draft"])
        assert L[0] == s["planted_L"][0], seed
        np.testing.assert_array_equal(amax[0], np.argmax(s["logits"][0], axis=1))
    for forced in (0, 16):
        s = synth.make_step(synth.params_for(4, V=3000, prefix=("fixed", 8)), 3, plant_L=forced)
        L, _ = oracle.spec_verify(s["logits"], s["draft"])
        assert L[0] == forced


def test_verify_brute_force():
    rng = np.random.Generator(np.random.PCG64(41))
    for _ in range(50):
        n, D, V = 3, 5, 4
        logits = rng.integers(0, 3, size=(n, D, V)).astype(np.float32)   # many ties
        draft = rng.integers(0, V, size=(n, D)).astype(np.int32)
        L, _ = oracle.spec_verify(logits, draft)
        for r in range(n):
            want = D
            for i in range(D):
                if int(np.argmax(logits[r, i])) != draft[r, i]:
                    want = i
                    break
            assert L[r] == want


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_kv_append_is_bitwise_and_bounded(dtype):
    rng = np.random.Generator(np.random.PCG64(51))
    n, D, Hq, Hkv, d = 3, 6, 4, 2, 8
    q, kb, vb, kc, vc, prefix = _random_step(rng, n, D, Hq, Hkv, d, [5, 0, 9], dtype, cap=16)
    acc = np.array([2, 6, 0], np.int32)
    kc2, vc2, p2, err = oracle.kv_append(kc, vc, prefix, kb, vb, acc)
    assert err == 0 and p2.tolist() == [7, 6, 9]
    for it in range(n):
        P, L = int(prefix[it]), int(acc[it])
        np.testing.assert_array_equal(kc2[it, :, P:P + L], np.swapaxes(kb[it, :L], 0, 1))
        np.testing.assert_array_equal(vc2[it, :, P:P + L], np.swapaxes(vb[it, :L], 0, 1))
        untouched_k = np.ones(kc.shape[2], bool)
        untouched_k[P:P + L] = False
        bits = lambda a: np.ascontiguousarray(a).view(np.uint8)
        np.testing.assert_array_equal(bits(kc2[it][:, untouched_k]), bits(kc[it][:, untouched_k]))
        np.testing.assert_array_equal(bits(vc2[it][:, untouched_k]), bits(vc[it][:, untouched_k]))
    # Overflow: that item is skipped and the error word is set.
    kc3, vc3, p3, err = oracle.kv_append(kc, vc, np.array([12, 0, 0], np.int32), kb, vb, None)
    assert err == 1 and p3.tolist() == [12, 6, 6]
    assert kc3[0].view(np.uint8).tobytes() == kc[0].view(np.uint8).tobytes()


def test_kv_append_fp8_bytes():
    """E4M3 caches are appended byte for byte (any code, NaN codes included)."""
    rng = np.random.Generator(np.random.PCG64(52))
    n, D, Hkv, d, cap = 2, 5, 2, 16, 32
    kc = rng.integers(0, 256, size=(n, Hkv, cap, d), dtype=np.uint8)
    vc = rng.integers(0, 256, size=(n, Hkv, cap, d), dtype=np.uint8)
    kb = rng.integers(0, 256, size=(n, D, Hkv, d), dtype=np.uint8)
    vb = rng.integers(0, 256, size=(n, D, Hkv, d), dtype=np.uint8)
    prefix = np.array([3, 27], np.int32)
    kc2, vc2, p2, err = oracle.kv_append(kc, vc, prefix, kb, vb, np.array([5, 5], np.int32))
    assert err == 0 and p2.tolist() == [8, 32]
    for it in range(n):
        P = int(prefix[it])
        np.testing.assert_array_equal(kc2[it, :, P:P + D], np.swapaxes(kb[it], 0, 1))
        np.testing.assert_array_equal(vc2[it, :, P:P + D], np.swapaxes(vb[it], 0, 1))
        keep = np.ones(cap, bool)
        keep[P:P + D] = False
        np.testing.assert_array_equal(kc2[it][:, keep], kc[it][:, keep])
        np.testing.assert_array_equal(vc2[it][:, keep], vc[it][:, keep])


# ---------------------------------------------------------------------------
# Split-K merge rule (online softmax normaliser, Milakov and Gimelshein 2018):
# any partition of the keys, merged in order, equals the unsplit softmax.
# ---------------------------------------------------------------------------

def _direct_softmax_sum(s, v):
    w = np.exp(s - s.max())
    return (w[:, None] * v).sum(axis=0) / w.sum()


@pytest.mark.parametrize("seed", range(6))
def test_merge_of_any_partition_equals_unsplit(seed):
    rng = np.random.default_rng(seed)
    n, d = int(rng.integers(5, 400)), 32
    s = rng.standard_normal(n) * float(rng.choice([0.5, 4.0, 40.0]))
    v = rng.standard_normal((n, d))
    want = _direct_softmax_sum(s, v)
    # random contiguous ranges, one of them empty
    cuts = np.sort(rng.choice(np.arange(1, n), size=min(6, n - 1), replace=False))
    bounds = [0] + cuts.tolist() + [n]
    ranges = [(a, b) for a, b in zip(bounds[:-1], bounds[1:])] + [(n, n)]
    parts = [oracle.softmax_partial(s[a:b], v[a:b].reshape(b - a, d)) for a, b in ranges]
    got = oracle.merge_partials(parts)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    # the order of merging changes only the rounding
    np.testing.assert_allclose(oracle.merge_partials(parts[::-1]), want, rtol=0, atol=1e-12)


def test_single_partial_is_the_softmax_and_empty_is_neutral():
    rng = np.random.default_rng(7)
    s = rng.standard_normal(50) * 3
    v = rng.standard_normal((50, 8))
    m, l, o = oracle.softmax_partial(s, v)
    assert m == s.max()
    np.testing.assert_allclose(l, np.exp(s - s.max()).sum(), rtol=1e-15)
    np.testing.assert_allclose(o, _direct_softmax_sum(s, v), atol=1e-13)
    me, le, oe = oracle.softmax_partial(np.zeros(0), np.zeros((0, 8)))
    assert me == -np.inf and le == 0.0 and not oe.any()
    np.testing.assert_array_equal(oracle.merge_partials([(m, l, o), (me, le, oe)]),
                                  oracle.merge_partials([(m, l, o)]))


def test_merge_matches_split_attention_rows():
    """A block-attention row computed by the oracle equals the merge of partials
    over a split of its keys (cache part, block part)."""
    p = synth.params_for(1, n_items=1, D=4, prefix=("fixed", 40), Hq=2, Hkv=1, d=64)
    st = synth.make_step(p, 11)
    out = oracle.attention(st["q"], st["k_blk"], st["v_blk"], st["k_cache"], st["v_cache"],
                           st["prefix"], oracle.BIDIR)
    q = st["q"][0, 2, 1].astype(np.float64)
    K = np.concatenate([st["k_cache"][0, 0, :40], st["k_blk"][0, :, 0]]).astype(np.float64)
    Vv = np.concatenate([st["v_cache"][0, 0, :40], st["v_blk"][0, :, 0]]).astype(np.float64)
    sc = K @ q / np.sqrt(64)
    parts = [oracle.softmax_partial(sc[a:b], Vv[a:b]) for a, b in ((0, 17), (17, 40), (40, 44))]
    np.testing.assert_allclose(oracle.merge_partials(parts), out[0, 2, 1], atol=1e-12)


# ---------------------------------------------------------------------------
# LM-head logits (vocabulary projection of the block's final hidden states).
# ---------------------------------------------------------------------------

def test_lm_head_logits_brute_force_and_unit_weights():
    rng = np.random.default_rng(3)
    n_req, D, H, V = 2, 3, 64, 37
    hidden = synth.f32_to_bf16_bits(rng.standard_normal((n_req, D, H), dtype=np.float32))
    weight = synth.f32_to_bf16_bits(rng.standard_normal((V, H), dtype=np.float32))
    got = oracle.lm_head_logits(hidden, weight)
    hf = synth.bf16_bits_to_f32(hidden).astype(np.float64)
    wf = synth.bf16_bits_to_f32(weight).astype(np.float64)
    for r in range(n_req):
        for i in range(D):
            for v in range(V):
                want = math.fsum(float(hf[r, i, h]) * float(wf[v, h]) for h in range(H))
                assert abs(got[r, i, v] - want) <= 1e-12 * (1 + abs(want))
    # unit weight rows pick single hidden components exactly
    unit = np.zeros((H, H), np.float32)
    unit[np.arange(H), (np.arange(H) * 7) % H] = 1.0
    picked = oracle.lm_head_logits(hidden, synth.f32_to_bf16_bits(unit))
    np.testing.assert_array_equal(picked, hf[:, :, (np.arange(H) * 7) % H])


def test_lm_head_planted_tokens_win():
    """The generator's planted weight rows (a scaled copy of a masked row's hidden
    state) give that row a logit near the gain, far above the rest."""
    st = synth.lmhead_step(2)
    logits = oracle.lm_head_logits(st["hidden"], st["weight"])
    for r, i, v_star in st["planted"]:
        assert int(np.argmax(logits[r, i])) == v_star
        assert logits[r, i, v_star] > 12.0


# ---------------------------------------------------------------------------
# FP8 (OCP E4M3) KV cache variant of the block attention.
# ---------------------------------------------------------------------------

def test_fp8_e4m3_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.fp8_e4m3_decode(codes)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2  # 0x7F and 0xFF
    np.testing.assert_array_equal(got[~nan], want[~nan])
    assert got[0x38] == 1.0 and got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


@pytest.mark.parametrize("mode", [oracle.BIDIR, oracle.CAUSAL])
def test_attention_fp8kv_equals_attention_on_dequantized_values(mode):
    """With power-of-two scales every dequantized key / value is exact in fp32, so the
    FP8-KV oracle must agree with the plain oracle fed those fp32 values."""
    p = synth.params_for(1, n_items=2, D=5, prefix=("list", [37, 70]), Hq=4, Hkv=2, d=64, dtype=synth.FP8KV)
    st = synth.make_step(p, 21)
    ks = np.exp2(np.round(np.log2(st["k_scale"]))).astype(np.float32)
    vs = np.exp2(np.round(np.log2(st["v_scale"]))).astype(np.float32)
    got = oracle.attention_fp8kv(st["q"], st["k_blk"], st["v_blk"], st["k_cache"], st["v_cache"], ks, vs,
                                 st["prefix"], mode)
    dec = lambda a, sc, axis_g: (oracle.fp8_e4m3_decode(a) * np.expand_dims(sc, axis=tuple(
        i for i in range(a.ndim) if i not in (0, axis_g)))).astype(np.float32)
    qf = synth.bf16_bits_to_f32(st["q"])
    kc = dec(st["k_cache"], ks, 1)
    vc = dec(st["v_cache"], vs, 1)
    kb = dec(st["k_blk"], ks, 2)
    vb = dec(st["v_blk"], vs, 2)
    # NaN canaries past the prefix stay NaN in the dequantized cache and must not be read
    want = oracle.attention(qf, kb, vb, kc, vc, st["prefix"], mode)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_quad_fp8kv_equals_quad_on_dequantized_values():
    """The quadratic mask over an E4M3 cache (power-of-two scales, so every
    dequantized value is exact in fp32) equals the plain quadratic oracle."""
    B = 4
    p = dict(synth.QUAD_CONFIGS[2], n_items=2, Hq=4, Hkv=2, d=64, B=B, prefix=("list", [21, 66]), dtype=synth.FP8KV)
    st = synth.make_quad_step(p, 31)
    ks = np.exp2(np.round(np.log2(st["k_scale"]))).astype(np.float32)
    vs = np.exp2(np.round(np.log2(st["v_scale"]))).astype(np.float32)
    got = oracle.attention_fp8kv(st["q"], st["k_blk"], st["v_blk"], st["k_cache"], st["v_cache"], ks, vs,
                                 st["prefix"], oracle.QUAD, B=B)
    dec = lambda a, sc, axis_g: (oracle.fp8_e4m3_decode(a) * np.expand_dims(sc, axis=tuple(
        i for i in range(a.ndim) if i not in (0, axis_g)))).astype(np.float32)
    want = oracle.attention_quad(synth.bf16_bits_to_f32(st["q"]), dec(st["k_blk"], ks, 2), dec(st["v_blk"], vs, 2),
                                 dec(st["k_cache"], ks, 1), dec(st["v_cache"], vs, 1), st["prefix"], B)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Two-stream training attention (Fast-dVLM write-up, sections 4.1, 4.3, 4.4;
# summary page Fig. 3): the oracle against (a) a dense mask built turn by turn
# from the three mask rules plus auto-truncation, evaluated by SDPA, and (b)
# the decode-time forms: causal prefill of the clean stream, and a denoise
# step per noisy block whose cache is the clean stream before it.
# ---------------------------------------------------------------------------

def _two_stream_dense_mask(Lc, Ln, spans, D):
    """[L][L] mask, L = Lc + Ln, from the rules: clean rows causal over clean keys
    (M_C2C); for each response (start c, length m) at noisy offset o, blocks of D
    from its start with the last one cut at c + m (auto-truncation); a noisy block
    sees clean keys before its start (M_N2C) and itself (M_N2N)."""
    L = Lc + Ln
    mask = np.zeros((L, L), bool)
    mask[:Lc, :Lc] = np.tril(np.ones((Lc, Lc), bool))
    o = 0
    for c, m in spans:
        for k0 in range(0, m, D):
            k1 = min(k0 + D, m)
            rows = slice(Lc + o + k0, Lc + o + k1)
            mask[rows, :c + k0] = True
            mask[rows, Lc + o + k0:Lc + o + k1] = True
        o += m
    return mask


@pytest.mark.parametrize("cfg_seed", [0, 1, 2])
def test_two_stream_matches_dense_mask(cfg_seed):
    p = dict(synth.TWO_STREAM_CONFIGS[2])
    st = synth.make_two_stream(p, 500 + cfg_seed)
    Lc, Ln = st["Lc"], st["Ln"]
    out = oracle.two_stream_attention(st["q"], st["k"], st["v"], st["spans"], st["n_spans"], Lc, p["D"])
    L, G = Lc + Ln, p["Hq"] // p["Hkv"]
    for it in range(p["n_seq"]):
        sp = [tuple(x) for x in st["spans"][it, :st["n_spans"][it]]]
        mask = _two_stream_dense_mask(Lc, Ln, sp, p["D"])
        live = mask.any(axis=1)
        Q = np.swapaxes(_widen(st["q"][it]), 0, 1)                  # [Hq][L][d]
        K = _widen(st["k"][it][:, :L])                               # [Hkv][L][d]
        V = _widen(st["v"][it][:, :L])                               # [Hkv][L][d]
        ref = _sdpa(Q[:, live], K, V, mask[live], G)
        np.testing.assert_allclose(out[it][live], np.swapaxes(ref, 0, 1), rtol=0, atol=1e-12)
        assert np.all(out[it][~live] == 0.0)                         # noisy padding sees nothing


def test_two_stream_equals_prefill_and_per_block_denoise():
    """Clean rows = causal prefill (CAUSAL block steps over chunks of the clean
    stream); each noisy block = a BIDIR step whose cache is the clean stream
    before the block and whose block is that noisy block (truncated blocks
    included)."""
    p = dict(synth.TWO_STREAM_CONFIGS[2])
    st = synth.make_two_stream(p, 77)
    Lc, Ln, D = st["Lc"], st["Ln"], p["D"]
    out = oracle.two_stream_attention(st["q"], st["k"], st["v"], st["spans"], st["n_spans"], Lc, D)
    for it in range(p["n_seq"]):
        Kseq = np.swapaxes(st["k"][it], 0, 1)                        # [cap][Hkv][d]
        Vseq = np.swapaxes(st["v"][it], 0, 1)                        # [cap][Hkv][d]
        kc, vc = st["k"][it:it + 1], st["v"][it:it + 1]
        for c0 in range(0, Lc, 7):                                    # clean chunks of 7 positions
            c1 = min(c0 + 7, Lc)
            ref = oracle.attention(st["q"][it:it + 1, c0:c1], Kseq[None, c0:c1], Vseq[None, c0:c1], kc, vc,
                                   np.array([c0], np.int32), CAUSAL)
            np.testing.assert_allclose(out[it:it + 1, c0:c1], ref, rtol=0, atol=1e-12)
        o = 0
        for c, m in st["spans"][it, :st["n_spans"][it]]:
            for k0 in range(0, m, D):
                k1 = min(k0 + D, m)
                rows = slice(Lc + o + k0, Lc + o + k1)
                ref = oracle.attention(st["q"][it:it + 1, rows], Kseq[None, rows], Vseq[None, rows], kc, vc,
                                       np.array([c + k0], np.int32), BIDIR)
                np.testing.assert_allclose(out[it:it + 1, rows], ref, rtol=0, atol=1e-12)
            o += m


# ---------------------------------------------------------------------------
# Fragile commit decisions (within 1e-4 of a tie in the oracle's fp64 values):
# the committed counts per config are reproducible from the oracle alone, and
# bounded.  Bounds: excluded decisions (rank | tau) at most 2% of the decisions
# of a block loop (at least 2 allowed).  Margin-only rows (still compared
# exactly: both sides take the argmax on the raw fp32 logits) at most 25%: with
# N(0, 4) logits over ~152k tokens the top two probabilities differ by less
# than 1e-4 in roughly one row in ten.
# ---------------------------------------------------------------------------

def test_fragile_counts_match_the_committed_artefact_and_stay_bounded():
    import acceptance
    with open(os.path.join(GOLDEN, "fragile_counts.json")) as f:
        stored = json.load(f)["configs"]
    for cfg in (1, 2, 3, 5):
        got = acceptance.summarize(cfg)
        assert got == stored[str(cfg)], (cfg, got, stored[str(cfg)])
        for part in ("first_step", "block_loop"):
            c = got[part]
            assert c["excluded"] <= max(2, 0.02 * c["decisions"]), (cfg, part, c)
            assert c["margin"] <= max(2, 0.25 * c["decisions"]), (cfg, part, c)
        assert got["block_loop"]["steps"] <= got["S"]


def test_fragile_rule_flags_each_kind_of_near_tie():
    """Hand-made confidences: a tau near-tie, a k-boundary near-tie, a runner-up
    near-tie; and nothing fragile when every gap is wide."""
    import acceptance
    masked = np.array([1, 1, 1, 1, 0], bool)
    conf = np.array([0.90005, 0.5, 0.49995, 0.1, np.nan])
    p2 = np.array([0.01, 0.49995, 0.2, 0.05, np.nan])
    f = acceptance.fragile(conf, p2, masked, k=1, tau=0.9)
    assert f["tau"] == {0} and f["rank"] == set() and f["margin"] == {1}
    f = acceptance.fragile(conf, p2, masked, k=2, tau=0.95)
    assert f["rank"] == {1, 2} and f["tau"] == set()
    wide = np.array([0.9, 0.6, 0.3, 0.1, np.nan])
    f = acceptance.fragile(wide, np.array([0.01, 0.2, 0.1, 0.05, np.nan]), masked, k=2, tau=0.95)
    assert not (f["rank"] or f["tau"] or f["margin"])
