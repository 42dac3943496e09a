"""GPU parity: libbd.so (through its C ABI) against the fp64 CPU oracle.

Bars:
  * bf16 / fp32 attention: max |gpu - oracle| <= 2e-2 and, per item,
    ||gpu - oracle||_2 / ||oracle||_2 <= 1e-2.
  * confidences: |gpu - oracle| <= 1e-5 absolute.
  * greedy tokens, committed sets, accepted lengths, appended bytes: exact.
    A commit decision is excluded (and counted) only where the oracle's own
    fp64 values put it within 1e-4 of a tie: the k-th / (k+1)-th confidence
    boundary, or the threshold tau (tests/acceptance.py; the counts per
    config are in tests/golden/fragile_counts.json).  The GPU's committed set
    must in addition equal the rule applied exactly to the GPU's own
    confidences.
  * every buffer the library writes sits between canary bands that must be
    intact after the test, and outputs start poisoned.
"""

import json
import os
import sys
import zlib

import numpy as np
import pytest

import acceptance
import oracle
import synth
from synth import BF16, BIDIR, CAUSAL, F32, FP8KV, QUAD

pytestmark = pytest.mark.gpu

ATTN_MAX_ABS = 2e-2
ATTN_REL = 1e-2
CONF_ABS = 1e-5
GUARD = 4096  # canary bytes on each side of every buffer the library writes

with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "fragile_counts.json")) as _f:
    FRAGILE_COUNTS = json.load(_f)["configs"]

_LIVE = []  # guarded buffer sets created by the running test


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    from vlm_decoding_amd import bd, step  # raises if libbd.so is missing
    return dict(torch=torch, bd=bd, step=step)


@pytest.fixture(autouse=True)
def _guards_intact():
    """After every test: no buffer the library wrote may have been written past its ends."""
    _LIVE.clear()
    yield
    damaged = []
    for g in _LIVE:
        damaged += g.damaged()
    _LIVE.clear()
    assert not damaged, "guard bands overwritten: %s" % damaged


def _ds(dev, st, **kw):
    """DeviceStep with canary bands around every buffer the library writes."""
    ds = dev["step"].DeviceStep(st, guard_bytes=GUARD, **kw)
    _LIVE.append(ds.gb)
    return ds


def _guarded(dev):
    g = dev["step"].GuardedBuffers("cuda", GUARD)
    _LIVE.append(g)
    return g


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _out_host(dev, ds):
    dev["torch"].cuda.synchronize()
    a = ds.out.cpu().numpy()
    if ds.dtype in (BF16, FP8KV):  # E4M3 K/V attention writes bf16 outputs
        return synth.bf16_bits_to_f32(a.view(np.uint16)).astype(np.float64)
    return a.astype(np.float64)


def _check_attention(got, ref, label):
    assert np.all(np.isfinite(got)), label + ": non-finite output"
    err = np.abs(got - ref)
    max_abs = float(err.max())
    rels = [float(np.linalg.norm((got[i] - ref[i]).ravel()) / np.linalg.norm(ref[i].ravel()))
            for i in range(ref.shape[0])]
    _say("%s: max_abs=%.3g max_rel_l2=%.3g" % (label, max_abs, max(rels)))
    assert max_abs <= ATTN_MAX_ABS, (label, max_abs)
    assert max(rels) <= ATTN_REL, (label, max(rels))


def _run_attention(dev, step_np, mode=None, label="", balanced=False):
    ds = _ds(dev, step_np, balanced=balanced)
    p = step_np["params"]
    mode = p["mode"] if mode is None else mode
    _say("attention %s n=%d D=%d Hq=%d Hkv=%d d=%d dtype=%d mode=%d prefix=%s balanced=%s" % (
        label, p["n_items"], p["D"], p["Hq"], p["Hkv"], p["d"], p["dtype"], mode,
        np.unique(step_np["prefix"])[:8].tolist(), balanced))
    ds.attn(mode=mode)
    got = _out_host(dev, ds)
    ref = _reference(step_np, mode)
    _check_attention(got, ref, label)
    return ds, got


def _reference(step_np, mode, items=None):
    """The oracle's attention for the step (all items, or the listed ones)."""
    p = step_np["params"]
    sl = (lambda a: a) if items is None else (lambda a: np.ascontiguousarray(a[items]))
    args = [sl(step_np[k]) for k in ("q", "k_blk", "v_blk", "k_cache", "v_cache")]
    if p["dtype"] == FP8KV:
        return oracle.attention_fp8kv(*args, sl(step_np["k_scale"]), sl(step_np["v_scale"]), sl(step_np["prefix"]),
                                      mode, B=p.get("B"))
    if mode == QUAD:
        return oracle.attention_quad(*args, sl(step_np["prefix"]), p["B"])
    return oracle.attention(*args, sl(step_np["prefix"]), mode)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_attention_configs(dev, cfg):
    """Every configuration at its full size, every output element against the oracle."""
    _run_attention(dev, synth.config_step(cfg), label="cfg%d" % cfg)


ATTN_CASES = [
    # (label, overrides)  -- small shapes spanning several tiles and ragged tails
    ("tail_only_P0", dict(prefix=("fixed", 0))),
    ("P_lt_tile", dict(prefix=("fixed", 37))),
    ("P_exact_tiles", dict(prefix=("fixed", 256))),
    ("P_ragged", dict(prefix=("list", [1, 63, 64, 65, 200, 511, 640, 1000]), n_items=8)),
    ("P_ragged32", dict(prefix=("list", [31, 32, 33, 95, 96, 97, 1023, 1024]), n_items=8)),
    ("D64_three_tail_tiles", dict(D=64, prefix=("list", [31, 94]), n_items=2)),
    ("D1_decode", dict(D=1, prefix=("fixed", 300))),
    ("D3_rows_pad", dict(D=3, prefix=("fixed", 129))),
    ("D64_two_row_blocks", dict(D=64, prefix=("fixed", 130))),
    ("G7_rows224", dict(Hq=28, Hkv=4, D=32, prefix=("list", [70, 500]), n_items=2)),
    ("d64_bf16", dict(d=64, prefix=("fixed", 333))),
    ("many_items", dict(n_items=40, prefix=("fixed", 150))),
    # capacities that are not multiples of 64 (nor of 8): each (item, KV head)'s
    # cache rows then start at an odd multiple of the row size
    ("cap1016", dict(prefix=("fixed", 1000), cap=1016)),
    ("cap1001", dict(prefix=("fixed", 1000), cap=1001)),
    ("cap1019_ragged", dict(prefix=("list", [1, 63, 517, 1000]), n_items=4, cap=1019)),
    ("cap25_short", dict(prefix=("list", [0, 7, 24]), n_items=3, cap=25)),
]


@pytest.mark.parametrize("mode", [BIDIR, CAUSAL])
@pytest.mark.parametrize("label,ov", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
def test_attention_edge_cases(dev, label, ov, mode):
    base = dict(n_items=2, Hq=16, Hkv=2, d=128, dtype=BF16, D=16, n_masked=8, V=1000, plant=None)
    base.update(ov)
    p = synth.params_for(3, **base)
    _run_attention(dev, synth.make_step(p, seed=zlib.crc32(label.encode()) % 10000), mode=mode, label=label)


# The balanced plan of ragged batches (BD_PLAN_BALANCED): every item's split
# count comes from the device-side prefix lengths.  The 7B batch (8 ragged
# items, 8-wave workgroups) in bf16 and over an E4M3 cache, the uniform 3B step
# (the plan reduces to the plain one), and ragged edge cases in both modes.
@pytest.mark.parametrize("cfg,dtype", [(5, BF16), (5, FP8KV), (3, BF16)])
def test_attention_balanced_configs(dev, cfg, dtype):
    _run_attention(dev, synth.config_step(cfg, dtype=dtype), label="balanced_cfg%d_dtype%d" % (cfg, dtype),
                   balanced=True)


BALANCED_CASES = [
    ("P_ragged", dict(prefix=("list", [1, 63, 64, 65, 200, 511, 640, 1000]), n_items=8)),
    ("P_ragged_wide", dict(prefix=("list", [0, 4096, 31, 2050, 17, 3000]), n_items=6)),
    ("two_items_4133_9", dict(n_items=2, prefix=("list", [4133, 9]))),
    ("G7_rows224", dict(Hq=28, Hkv=4, D=32, prefix=("list", [70, 2500, 900]), n_items=3)),
    ("many_items_64", dict(n_items=64, prefix=("list", [(37 * i) % 700 for i in range(64)]))),
    ("d64", dict(d=64, prefix=("list", [333, 1, 1500]), n_items=3)),
    ("fp8_ragged", dict(dtype=FP8KV, prefix=("list", [0, 63, 64, 1000, 2049]), n_items=5)),
]


@pytest.mark.parametrize("mode", [BIDIR, CAUSAL])
@pytest.mark.parametrize("label,ov", BALANCED_CASES, ids=[c[0] for c in BALANCED_CASES])
def test_attention_balanced_edge_cases(dev, label, ov, mode):
    base = dict(n_items=2, Hq=16, Hkv=2, d=128, dtype=BF16, D=16, n_masked=8, V=1000, plant=None)
    base.update(ov)
    p = synth.params_for(3, **base)
    _run_attention(dev, synth.make_step(p, seed=zlib.crc32(("bal" + label).encode()) % 10000), mode=mode,
                   label="balanced_" + label, balanced=True)


def test_attention_balanced_deterministic_and_quad(dev):
    """Repeated balanced calls are bitwise identical; the quadratic mode with ragged
    prefixes under the balanced plan matches the oracle."""
    torch = dev["torch"]
    p = synth.params_for(5, n_items=4, prefix=("list", [300, 5000, 64, 2048]), V=1000, plant=None)
    s = synth.make_step(p, seed=55)
    ds = _ds(dev, s, balanced=True)
    ds.attn()
    torch.cuda.synchronize()
    first = ds.out.clone()
    for _ in range(3):
        ds.out.zero_()
        ds.attn()
    torch.cuda.synchronize()
    assert torch.equal(first, ds.out)
    _check_attention(_out_host(dev, ds), _reference(s, p["mode"]), "balanced_7b_ragged")
    q = dict(synth.QUAD_CONFIGS[2], B=16, n_items=4, prefix=("list", [0, 95, 96, 1200]))
    _run_attention(dev, synth.make_quad_step(q, 66), label="balanced_quad_B16", balanced=True)


@pytest.mark.parametrize("n_items", [64, 65])
def test_attention_balanced_at_the_item_limit(dev, n_items):
    """The balanced plan takes one lane per item: 64 ragged items (empty prefixes
    and prefixes shorter than a tile among them) use it, 65 fall back to the plain
    plan.  Every item of the output against the oracle."""
    rng = np.random.default_rng(640 + n_items)
    pre = rng.integers(0, 2400, size=n_items)
    pre[::9] = 0
    pre[1::11] = rng.integers(1, 32, size=len(pre[1::11]))
    p = synth.params_for(3, n_items=n_items, D=16, prefix=("list", pre.tolist()), V=1000, n_masked=8, plant=None)
    _run_attention(dev, synth.make_step(p, 640 + n_items), label="balanced_%d_items" % n_items, balanced=True)


# Few items with long prefixes: the plan gives such calls 32 or 64 splits per
# unit (every workgroup on a CU of its own) and merges them with the 32-slot
# merge instance or its form with eight split waves of 8 slots.  Ragged
# prefixes give units with fewer splits than the plan's maximum (with 4096 and
# 300, the short unit's few splits all fall to the first split wave).
FEW_ITEM_CASES = [
    ("one_item_4096_64_splits", dict(n_items=1, prefix=("fixed", 4096))),
    ("two_items_ragged_64_splits", dict(n_items=2, prefix=("list", [4096, 2050]))),
    ("two_items_4096_300_64_splits", dict(n_items=2, prefix=("list", [4096, 300]))),
    ("two_items_4133_tail", dict(n_items=2, prefix=("list", [4133, 4127]))),
    ("four_items_32_splits", dict(n_items=4, prefix=("list", [2048, 1100, 31, 2047]))),
    ("one_item_fp8_32_splits", dict(n_items=1, prefix=("fixed", 4096), dtype=FP8KV)),
]


@pytest.mark.parametrize("mode", [BIDIR, CAUSAL])
@pytest.mark.parametrize("label,ov", FEW_ITEM_CASES, ids=[c[0] for c in FEW_ITEM_CASES])
def test_attention_few_items_many_splits(dev, label, ov, mode):
    base = dict(Hq=16, Hkv=2, d=128, dtype=BF16, D=16, n_masked=8, V=1000, plant=None)
    base.update(ov)
    p = synth.params_for(3, **base)
    _run_attention(dev, synth.make_step(p, seed=zlib.crc32(label.encode()) % 10000), mode=mode, label=label)


# Paired halves: where two 4-wave workgroups would share every CU (d = 128,
# fixed split plan, more list slots than CUs), one 8-wave workgroup runs two
# adjacent list slots and combines them in LDS when both belong to one unit.
# Ragged prefixes give units with different split counts (pairs across unit
# boundaries, halves with nothing to stream, units whose only partial is one
# combined pair, written out directly); an odd list length leaves the last
# workgroup's second half empty; a plan sized for a much longer context than
# any prefix leaves whole workgroups empty.
PAIR_CASES = [
    ("ragged_40_items", dict(n_items=40, prefix=("list", [(0, 1, 31, 32, 33, 100, 500, 1000, 1500, 2047)[i % 10]
                                                          for i in range(40)])), 2048),
    ("odd_list_37_units", dict(n_items=37, Hq=8, Hkv=1, prefix=("list", [(53 * i) % 1000 for i in range(37)])), 1000),
    ("short_prefixes_long_plan", dict(n_items=36, prefix=("list", [(7 * i) % 70 for i in range(36)])), 4096),
    ("two_split_units", dict(n_items=64, prefix=("fixed", 40)), 128),
]


@pytest.mark.parametrize("dtype", [BF16, FP8KV])
@pytest.mark.parametrize("mode", [BIDIR, CAUSAL])
@pytest.mark.parametrize("label,ov,host_max", PAIR_CASES, ids=[c[0] for c in PAIR_CASES])
def test_attention_paired_halves(dev, label, ov, host_max, mode, dtype):
    base = dict(n_items=2, Hq=16, Hkv=2, d=128, dtype=dtype, D=16, n_masked=8, V=1000, plant=None,
                cap=host_max + 16)
    base.update(ov)
    p = synth.params_for(3, **base)
    st = synth.make_step(p, seed=zlib.crc32(("pair" + label).encode()) % 10000)
    _say("attention pair_%s n=%d Hq=%d Hkv=%d dtype=%d mode=%d max_prefix=%d" % (
        label, p["n_items"], p["Hq"], p["Hkv"], dtype, mode, host_max))
    ds = _ds(dev, st, max_prefix=host_max)
    ds.attn(mode=mode)
    _check_attention(_out_host(dev, ds), _reference(st, mode), "pair_" + label)


# Seeded random sweep over small shapes: dtype (bf16, E4M3 cache, fp32), mask
# mode (bidirectional, causal, quadratic), head layout, d, block length and
# ragged prefixes drawn together, and for about half the cases a plan sized
# for a longer context than any prefix (its surplus workgroups must exit and
# the rest must not read past a prefix: cache slots there hold NaN).
N_SWEEP = 32


def _sweep_case(i):
    rng = np.random.default_rng(5000 + i)

    def one_prefix():
        kind = int(rng.integers(0, 3))
        if kind == 0:
            return 0 if rng.random() < 0.5 else int(rng.integers(1, 40))
        if kind == 1:
            return int(rng.integers(1, 1300))
        return int(64 * rng.integers(1, 20) + rng.integers(-1, 2))  # at and around tile edges

    while True:
        dtype = int(rng.choice([BF16, BF16, FP8KV, F32]))
        mode = int(rng.choice([BIDIR, CAUSAL, QUAD]))
        d = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2, 4]))
        Hq = Hkv * int(rng.choice([1, 2, 3, 4, 7, 8]))
        n = int(rng.integers(1, 6))
        B = int(rng.integers(1, 11)) if mode == QUAD else None
        D = synth.quad_slot_count(B) if mode == QUAD else int(rng.integers(1, 65))
        prefix = [one_prefix() for _ in range(n)]
        host_max = max(prefix) + (int(rng.integers(1, 700)) if rng.random() < 0.5 else 0)
        if n * Hq * D * (max(prefix) + D) * d <= 1.5e8:  # keeps the fp64 oracle within seconds
            break
    balanced = bool(rng.random() < 0.5)  # drawn after the shape, so the shapes of the sweep stay put
    # the smallest capacity that holds the largest prefix plus one block
    p = dict(n_items=n, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, prefix=("list", prefix), cap=host_max + D)
    if mode == QUAD:
        st = synth.make_quad_step(dict(synth.QUAD_CONFIGS[2], B=B, **p), 5000 + i)
    else:
        st = synth.make_step(synth.params_for(3, D=D, mode=mode, n_masked=D // 2, V=1000, plant=None, **p),
                             5000 + i)
    return st, host_max, balanced


@pytest.mark.parametrize("i", range(N_SWEEP))
def test_attention_random_sweep(dev, i):
    st, host_max, balanced = _sweep_case(i)
    p = st["params"]
    label = "sweep%d" % i
    _say("attention %s n=%d D=%d B=%s Hq=%d Hkv=%d d=%d dtype=%d mode=%d prefix=%s max_prefix=%d cap=%d balanced=%s" % (
        label, p["n_items"], p["D"], p.get("B"), p["Hq"], p["Hkv"], p["d"], p["dtype"], p["mode"],
        st["prefix"].tolist(), host_max, st["cap"], balanced))
    ds = _ds(dev, st, max_prefix=host_max, balanced=balanced)
    ds.attn()
    _check_attention(_out_host(dev, ds), _reference(st, p["mode"]), label)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mode", [BIDIR, CAUSAL])
def test_attention_fp32_vector_path(dev, d, mode):
    p = synth.params_for(1, d=d, n_items=3, prefix=("list", [0, 70, 129]), Hq=6, Hkv=2, D=5)
    _run_attention(dev, synth.make_step(p, seed=77), mode=mode, label="fp32_d%d" % d)


def test_attention_deterministic_and_workspace_reuse(dev):
    """Bitwise-identical results over repeated calls on one workspace (the split
    merge runs in a fixed order and the ticket counters reset themselves)."""
    torch = dev["torch"]
    s = synth.config_step(3)
    ds = _ds(dev, s)
    ds.attn()
    torch.cuda.synchronize()
    first = ds.out.clone()
    for _ in range(3):
        ds.out.zero_()
        ds.attn()
    torch.cuda.synchronize()
    assert torch.equal(first, ds.out)


def test_layer_serial_graph_replays_match_eager(dev):
    """The step with one bd_attn_step per layer, captured in a HIP graph: every
    replay (with other eager work and synchronisations in between) reproduces the
    eager layer-serial results bit for bit, and those match the oracle."""
    torch = dev["torch"]
    p = synth.params_for(3, n_items=4, prefix=("list", [0, 100, 700, 2000]), V=3001, n_masked=8, plant=None)
    st = synth.make_step(p, 321)
    ds = _ds(dev, st)
    ds.reset_block_state()
    ds.layer_serial_step()
    torch.cuda.synchronize()
    ref = [ds.out.clone(), ds.masked.clone(), ds.tokens.clone(), ds.conf.clone()]
    _check_attention(_out_host(dev, ds), _reference(st, p["mode"]), "layer_serial")
    g = ds.capture_layer_serial()
    for r in range(3):
        ds.out.zero_()
        ds.masked.fill_(3)
        ds.attn()  # eager work between replays (the batched call) ...
        torch.cuda.synchronize()
        ds.out.zero_()
        g.replay()
        torch.cuda.synchronize()
        got = [ds.out, ds.masked, ds.tokens, ds.conf]
        for a, b in zip(got, ref):
            if a.dtype == torch.float32:  # conf holds NaN at unmasked slots: compare bits
                a, b = a.view(torch.int32), b.view(torch.int32)
            assert torch.equal(a, b), r


def test_attention_rejects_bad_arguments_before_launch(dev):
    bd = dev["bd"]
    ds = _ds(dev, synth.config_step(2))
    bad = bd.attn_desc(1, 8, 16, 2, 96, ds.cap, BF16, BIDIR, 1024)
    with pytest.raises(bd.BdError) as e:
        bd.bd_attn_step(bad, ds.q, ds.k_blk, ds.v_blk, ds.k_cache, ds.v_cache, ds.prefix, ds.out, ds.attn_ws)
    assert e.value.status == bd.BD_E_SHAPE


# ---------------------------------------------------------------------------
# Attention over an FP8 (E4M3) KV cache.  The bar is the bf16 one: E4M3 codes
# widen to bf16 exactly, so the GPU's arithmetic differs from the oracle's
# fp64 (on the same decoded values) only as the bf16 path's does.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cfg,mode", [(3, BIDIR), (4, CAUSAL), (5, BIDIR)])
def test_fp8kv_attention_configs(dev, cfg, mode):
    """The 3B long-context step, the 3B verify shape and the 7B batch at full size with
    an E4M3 cache, every output element against the oracle."""
    _run_attention(dev, synth.config_step(cfg, dtype=FP8KV), mode=mode, label="fp8kv_cfg%d" % cfg)


FP8_CASES = [
    # 64-key E4M3 tiles: prefixes around tile edges, tails of one and two tiles
    ("tail_only_P0", dict(prefix=("fixed", 0))),
    ("P_lt_tile", dict(prefix=("fixed", 37))),
    ("P_exact_tiles", dict(prefix=("fixed", 256))),
    ("P_ragged64", dict(prefix=("list", [1, 63, 64, 65, 127, 128, 129, 1000]), n_items=8)),
    ("P_ragged16", dict(prefix=("list", [15, 16, 17, 31, 33, 47, 49, 1023]), n_items=8)),
    ("D64_two_tail_tiles", dict(D=64, prefix=("list", [63, 126]), n_items=2)),
    ("D1_decode", dict(D=1, prefix=("fixed", 300))),
    ("D3_rows_pad", dict(D=3, prefix=("fixed", 129))),
    ("D64_two_row_blocks", dict(D=64, prefix=("fixed", 130))),
    ("G7_rows224", dict(Hq=28, Hkv=4, D=32, prefix=("list", [70, 500]), n_items=2)),
    ("d64", dict(d=64, prefix=("fixed", 333))),
    ("d64_ragged", dict(d=64, D=32, prefix=("list", [0, 64, 65, 700]), n_items=4)),
    ("many_items", dict(n_items=40, prefix=("fixed", 150))),
    # capacities that are not multiples of 64 (1003: not even of 2)
    ("cap1008", dict(prefix=("fixed", 990), cap=1008)),
    ("cap1003", dict(prefix=("fixed", 990), cap=1003)),
    ("cap1003_ragged", dict(prefix=("list", [0, 65, 500, 990]), n_items=4, cap=1003)),
]


@pytest.mark.parametrize("mode", [BIDIR, CAUSAL])
@pytest.mark.parametrize("label,ov", FP8_CASES, ids=[c[0] for c in FP8_CASES])
def test_fp8kv_attention_edge_cases(dev, label, ov, mode):
    base = dict(n_items=2, Hq=16, Hkv=2, d=128, dtype=FP8KV, D=16, n_masked=8, V=1000, plant=None)
    base.update(ov)
    p = synth.params_for(3, **base)
    _run_attention(dev, synth.make_step(p, seed=zlib.crc32(("fp8" + label).encode()) % 10000), mode=mode,
                   label="fp8kv_" + label)


def test_fp8kv_deterministic_append_and_reattend(dev):
    """Repeated calls are bitwise identical; the E4M3 block appended to the cache is
    its bytes exactly, and attention over the grown cache matches the oracle."""
    torch = dev["torch"]
    p = synth.params_for(3, n_items=3, dtype=FP8KV, D=16, prefix=("list", [100, 64, 1500]), V=1000,
                         n_masked=8, plant=None)
    s = synth.make_step(p, seed=4242)
    ds = _ds(dev, s)
    ds.attn()
    torch.cuda.synchronize()
    first = ds.out.clone()
    for _ in range(2):
        ds.out.zero_()
        ds.attn()
    torch.cuda.synchronize()
    assert torch.equal(first, ds.out)
    acc = np.array([16, 5, 0], np.int32)
    ds.append(n_accept=torch.from_numpy(acc).cuda())
    torch.cuda.synchronize()
    kc, vc, pref, err = oracle.kv_append(s["k_cache"], s["v_cache"], s["prefix"], s["k_blk"], s["v_blk"], acc)
    assert err == 0 and int(ds.dev_err.cpu()[0]) == 0
    np.testing.assert_array_equal(ds.prefix.cpu().numpy(), pref)
    assert ds.k_cache.cpu().numpy().tobytes() == kc.tobytes()
    assert ds.v_cache.cpu().numpy().tobytes() == vc.tobytes()
    # The same block queried again over the grown cache (the desc keeps max_prefix
    # as the bound of the split plan; the grown prefixes stay within the capacity).
    s2 = dict(s, k_cache=kc, v_cache=vc, prefix=pref)
    ds.attn()
    got = _out_host(dev, ds)
    ref = oracle.attention_fp8kv(s2["q"], s2["k_blk"], s2["v_blk"], kc, vc, s["k_scale"], s["v_scale"], pref, BIDIR)
    _check_attention(got, ref, "fp8kv_after_append")


@pytest.mark.parametrize("dtype,cap", [(BF16, 2072), (BF16, 2069), (FP8KV, 2080), (FP8KV, 2071)])
def test_append_and_reattend_unaligned_cap(dev, dtype, cap):
    """Append into caches whose capacity is not a multiple of 64 (2069 and 2071 not
    even of 8), up to the last slot; the grown caches are the oracle's bit for bit
    and attention over them matches the oracle."""
    torch = dev["torch"]
    p = synth.params_for(3, n_items=3, dtype=dtype, D=16, prefix=("list", [cap - 16, 1000, 77]), cap=cap, V=1000,
                         n_masked=8, plant=None)
    s = synth.make_step(p, seed=cap + dtype)
    ds = _ds(dev, s, max_prefix=cap)
    acc = np.array([16, 9, 1], np.int32)
    ds.append(n_accept=torch.from_numpy(acc).cuda())
    torch.cuda.synchronize()
    kc, vc, pref, err = oracle.kv_append(s["k_cache"], s["v_cache"], s["prefix"], s["k_blk"], s["v_blk"], acc)
    assert err == 0 and int(ds.dev_err.cpu()[0]) == 0
    np.testing.assert_array_equal(ds.prefix.cpu().numpy(), pref)
    assert pref[0] == cap
    assert ds.k_cache.cpu().numpy().tobytes() == kc.tobytes()
    assert ds.v_cache.cpu().numpy().tobytes() == vc.tobytes()
    ds.attn()
    got = _out_host(dev, ds)
    s2 = dict(s, k_cache=kc, v_cache=vc, prefix=pref)
    _check_attention(got, _reference(s2, BIDIR), "append_cap%d_dtype%d" % (cap, dtype))


# ---------------------------------------------------------------------------
# Quadratic self-speculative attention (BD_BLOCK_QUAD): B drafts, causal among
# themselves, then B groups of mask tokens, group g seeing drafts 0..g-1 and
# itself.  Same bar as the bf16 attention.
# ---------------------------------------------------------------------------

def test_quad_small_config(dev):
    _run_attention(dev, synth.quad_step(2), label="quad_small")


def test_quad_3b_sampled_items(dev):
    """The 3B quadratic step at its full size (36 layers, prefix 4096, B = 16, 152
    slots): the GPU computes every layer in the launch that bench.py times; the
    oracle checks three whole layers of it."""
    st = synth.quad_step(1)
    ds = _ds(dev, st)
    p = st["params"]
    _say("quad 3b: n=%d slots=%d B=%d" % (p["n_items"], p["D"], p["B"]))
    ds.attn()
    got = _out_host(dev, ds)
    items = [0, 17, 35]
    ref = _reference(st, QUAD, items=items)
    _check_attention(got[items], ref, "quad_3b_items")


QUAD_CASES = [
    ("B1", dict(B=1, prefix=("list", [0, 50, 64]))),
    ("B2_ragged", dict(B=2, prefix=("list", [31, 32, 33]))),
    ("B8_G7", dict(B=8, Hq=28, Hkv=4, prefix=("list", [70, 500, 1]))),
    ("B16_ragged", dict(B=16, n_items=4, prefix=("list", [0, 95, 96, 1200]))),
    ("B32_560_slots", dict(B=32, n_items=1, prefix=("fixed", 100))),
    ("d64", dict(B=6, d=64, prefix=("list", [333, 64, 0]))),
]


@pytest.mark.parametrize("label,ov", QUAD_CASES, ids=[c[0] for c in QUAD_CASES])
def test_quad_edge_cases(dev, label, ov):
    p = dict(synth.QUAD_CONFIGS[2])
    p.update(ov)
    _run_attention(dev, synth.make_quad_step(p, zlib.crc32(("quad" + label).encode()) % 10000), label="quad_" + label)


@pytest.mark.parametrize("dtype", [F32, FP8KV])
def test_quad_fp32_and_fp8kv(dev, dtype):
    """The quadratic mask on the fp32 vector path and on the E4M3 KV-cache path."""
    p = dict(synth.QUAD_CONFIGS[2], dtype=dtype, B=6, prefix=("list", [0, 129, 700]))
    if dtype == F32:
        p.update(Hq=6, Hkv=2, d=64)
    _run_attention(dev, synth.make_quad_step(p, 99 + dtype), label="quad_dtype%d" % dtype)


def test_quad_append_accepted_drafts(dev):
    """After a quadratic step the accepted drafts (slots 0..L-1 of the B (B + 3) / 2)
    join the cache; L > B is refused on the device."""
    torch = dev["torch"]
    B = 5
    st = synth.make_quad_step(dict(synth.QUAD_CONFIGS[2], B=B), 123)
    ds = _ds(dev, st)
    acc = np.array([B, 0, 3], np.int32)
    ds.append(n_accept=torch.from_numpy(acc).cuda())
    torch.cuda.synchronize()
    kc, vc, pref, err = oracle.kv_append(st["k_cache"], st["v_cache"], st["prefix"], st["k_blk"], st["v_blk"], acc)
    assert err == 0 and int(ds.dev_err.cpu()[0]) == 0
    np.testing.assert_array_equal(ds.prefix.cpu().numpy(), pref)
    assert ds.k_cache.cpu().numpy().view(np.uint16).tobytes() == kc.tobytes()
    assert ds.v_cache.cpu().numpy().view(np.uint16).tobytes() == vc.tobytes()
    ds.append(n_accept=torch.tensor([B + 1, 0, 0], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert int(ds.dev_err.cpu()[0]) == 1
    np.testing.assert_array_equal(ds.prefix.cpu().numpy(), pref)  # item 0 refused, the others add 0


# ---------------------------------------------------------------------------
# Two-stream training attention (bd_two_stream_attn): clean stream causal, each
# noisy response block sees the clean positions before it and itself; blocks
# are cut at response ends.  Same bar as the bf16 attention.
# ---------------------------------------------------------------------------

def _run_two_stream(dev, st, label, items=None):
    torch, bd = dev["torch"], dev["bd"]
    p = st["params"]
    n, L, Hq, d = st["q"].shape
    _say("two-stream %s n=%d Lc=%d Ln=%d D=%d Hq=%d Hkv=%d d=%d spans=%s" % (
        label, n, st["Lc"], st["Ln"], p["D"], Hq, p["Hkv"], d, st["n_spans"].tolist()))
    c = lambda a: torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if a.dtype == np.uint16 else a)).cuda()
    q, k, v, sp, ns = c(st["q"]), c(st["k"]), c(st["v"]), c(st["spans"]), c(st["n_spans"])
    g = _guarded(dev)
    out = g.make("out", q.shape, q.dtype, fill=dev["step"].POISON)
    desc = bd.two_stream_desc(n, st["Lc"], st["Ln"], st["cap"], p["D"], Hq, p["Hkv"], d, st["spans"].shape[1])
    ws = g.make("ws", (max(bd.bd_two_stream_workspace_bytes(desc), 16),), torch.uint8, fill=0)
    bd.bd_two_stream_attn(desc, q, k, v, sp, ns, out, ws)
    torch.cuda.synchronize()
    got = synth.bf16_bits_to_f32(out.cpu().numpy().view(np.uint16)).astype(np.float64)
    sel = list(range(n)) if items is None else items
    ref = oracle.two_stream_attention(*[np.ascontiguousarray(st[x][sel]) for x in ("q", "k", "v", "spans", "n_spans")],
                                      st["Lc"], p["D"])
    _check_attention(got[sel], ref, label)
    return got, (desc, q, k, v, sp, ns, out, ws)


def test_two_stream_small_config(dev):
    _run_two_stream(dev, synth.two_stream_step(2), "two_stream_small")


def test_two_stream_3b_training_shape_sampled(dev):
    """The 3B training shape (8 sequences, clean 2048 with 1024 vision tokens, noisy
    832, D = 32) in one launch; the oracle checks two whole sequences of it."""
    _run_two_stream(dev, synth.two_stream_step(1), "two_stream_3b", items=[0, 7])


TWO_STREAM_CASES = [
    ("no_noisy_prefill", dict(turns=[(10, 0)], vision=100)),
    ("one_response_exact_blocks", dict(turns=[(7, 32)], D=8)),
    ("D1", dict(D=1, turns=[(4, 9), (3, 5)])),
    ("D_larger_than_responses", dict(D=64, turns=[(4, 30), (3, 17)])),
    ("G7_rows", dict(Hq=14, Hkv=2, d=128, turns=[(20, 70), (8, 41)])),
    ("d128_long", dict(d=128, vision=300, turns=[(33, 250), (12, 77)], D=32)),
    ("empty_span_and_padding", dict(turns=[[(5, 0), (6, 23)], [(2, 40)]], D=16)),
    # 6 units (one sequence, one KV head, 1420 positions): 32 splits, the 32-slot merge
    ("few_units_32_splits", dict(n_seq=1, Hq=1, Hkv=1, d=128, vision=600, turns=[(20, 400)], D=16)),
    # L = 200 positions in a 224-slot array: the smallest capacity the ABI takes (a
    # multiple of 32), so the last tile ends at the array's end
    ("cap_odd_multiple_of_32", dict(vision=120, turns=[(20, 30)], cap_align=32)),
]


@pytest.mark.parametrize("label,ov", TWO_STREAM_CASES, ids=[c[0] for c in TWO_STREAM_CASES])
def test_two_stream_edge_cases(dev, label, ov):
    p = dict(synth.TWO_STREAM_CONFIGS[2])
    p.update(ov)
    st = synth.make_two_stream(p, zlib.crc32(("ts" + label).encode()) % 10000)
    _run_two_stream(dev, st, "two_stream_" + label)


# Seeded random sweep of two-stream shapes: 1-3 sequences with their own turn
# lists (empty prompts and empty responses included), block lengths from 1 to
# longer than every response, GQA layouts with 1-8 query heads per KV head.
N_TS_SWEEP = 16


def _two_stream_sweep_case(i):
    rng = np.random.default_rng(6000 + i)
    while True:
        n = int(rng.integers(1, 4))
        Hkv = int(rng.choice([1, 2]))
        Hq = Hkv * int(rng.choice([1, 2, 4, 7, 8]))
        d = int(rng.choice([64, 128]))
        D = int(rng.choice([1, 2, 5, 8, 16, 32, 48]))
        turns = [[(int(rng.integers(0, 40)), int(rng.choice([0, rng.integers(1, 20), rng.integers(20, 160)])))
                  for _ in range(int(rng.integers(1, 4)))] for _ in range(n)]
        p = dict(synth.TWO_STREAM_CONFIGS[2], n_seq=n, Hq=Hq, Hkv=Hkv, d=d, D=D,
                 vision=int(rng.integers(1, 200)), turns=turns)
        Lc = p["vision"] + max(sum(a + b for a, b in t) for t in turns)
        L = Lc + max(sum(b for _, b in t) for t in turns)
        if n * L * L * Hq * d <= 3e8:  # keeps the fp64 oracle within seconds
            return synth.make_two_stream(p, 6000 + i)


@pytest.mark.parametrize("i", range(N_TS_SWEEP))
def test_two_stream_random_sweep(dev, i):
    _run_two_stream(dev, _two_stream_sweep_case(i), "two_stream_sweep%d" % i)


def test_two_stream_deterministic(dev):
    torch, bd = dev["torch"], dev["bd"]
    st = synth.make_two_stream(dict(synth.TWO_STREAM_CONFIGS[2], n_seq=1, Hq=2, Hkv=1, vision=2000,
                                    turns=[(30, 500)], D=32), 11)
    _, args = _run_two_stream(dev, st, "two_stream_split")
    desc, q, k, v, sp, ns, out, ws = args
    first = out.clone()
    for _ in range(3):
        out.zero_()
        bd.bd_two_stream_attn(desc, q, k, v, sp, ns, out, ws)
    torch.cuda.synchronize()
    assert torch.equal(first, out)


# ---------------------------------------------------------------------------
# Confidence + commit
# ---------------------------------------------------------------------------

def _rule_commit(conf32, masked, k, tau):
    """Top-k by (conf desc, index asc) plus {conf > tau}, on the GPU's fp32 values."""
    idx = [i for i in range(len(masked)) if masked[i]]
    order = sorted(idx, key=lambda i: (-float(conf32[i]), i))
    take = set(order[:k]) | {i for i in idx if conf32[i] > np.float32(tau)}
    return take


def _compare_commit(dev, ds, p, masked_in, tokens_in, logits_np, label):
    """GPU confidence + commit outputs (in ``ds``) against the oracle on the same
    inputs.  Returns (fragile counts, oracle result)."""
    torch = dev["torch"]
    torch.cuda.synchronize()
    ref = oracle.confidence_commit(logits_np, masked_in, tokens_in, p["S"], p["tau"])
    frag = acceptance.step_fragility(logits_np, masked_in, p["S"], p["tau"], ref)
    g_conf = ds.conf.cpu().numpy()
    g_arg = ds.argmax.cpu().numpy()
    g_com = ds.committed.cpu().numpy()
    g_ncom = ds.n_committed.cpu().numpy()
    g_mask = ds.masked.cpu().numpy()
    g_tok = ds.tokens.cpu().numpy()
    for r in range(p["n_req"]):
        m = masked_in[r].astype(bool)
        nm = int(m.sum())
        k = min(-(-p["D"] // p["S"]), nm)
        assert np.all(np.isnan(g_conf[r][~m])) and np.all(g_arg[r][~m] == -1)
        if nm:
            err = np.abs(g_conf[r][m].astype(np.float64) - ref["conf"][r][m])
            assert err.max() <= CONF_ABS, (label, r, err.max())
            np.testing.assert_array_equal(g_arg[r][m], ref["argmax"][r][m])  # margin rows included
        # The GPU applies the rule exactly to its own fp32 confidences ...
        own = _rule_commit(g_conf[r], m, k, p["tau"])
        assert set(np.nonzero(g_com[r])[0].tolist()) == own, (label, r)
        # ... and agrees with the oracle wherever the decision is not within 1e-4 of a tie.
        excl = frag[r]["rank"] | frag[r]["tau"]
        for i in range(p["D"]):
            if i in excl:
                continue
            assert g_com[r, i] == ref["committed"][r, i], (label, r, i)
            assert g_mask[r, i] == ref["masked"][r, i]
            assert g_tok[r, i] == ref["tokens"][r, i]
        assert g_ncom[r] == int(g_com[r].sum())
        untouched = ~m
        np.testing.assert_array_equal(g_tok[r][untouched], tokens_in[r][untouched])
        np.testing.assert_array_equal(g_mask[r][untouched], 0)
    return acceptance.counts(frag), ref


@pytest.mark.parametrize("cfg", [1, 2, 3, 5])
def test_confidence_commit_configs(dev, cfg):
    s = synth.config_step(cfg)
    p = s["params"]
    _say("confidence_commit cfg%d n_req=%d D=%d V=%d" % (cfg, p["n_req"], p["D"], p["V"]))
    ds = _ds(dev, s)
    ds.confidence_commit()
    c, _ = _compare_commit(dev, ds, p, s["masked"], s["tokens"], s["logits"], "cfg%d" % cfg)
    _say("cfg%d fragile decisions: %s" % (cfg, c))
    want = FRAGILE_COUNTS[str(cfg)]["first_step"]
    assert {k: c[k] for k in ("margin", "rank", "tau", "excluded")} == \
        {k: want[k] for k in ("margin", "rank", "tau", "excluded")}


@pytest.mark.parametrize("cfg", [1, 2, 3, 5])
def test_block_loop_on_own_state(dev, cfg):
    """The whole denoising loop of one block on the GPU's own state (DiffusionVL
    notes, cached block decoding and Algorithm 1): the GPU's masked / tokens are
    never reset between steps; each step gets the next seeded logits.  After
    every step the GPU's decisions match the oracle's on the same state (fragile
    ones excluded), its trajectory equals the oracle's own loop unless a counted
    fragile decision went the other way, committed tokens never change, each step
    commits at least min(k, |M|), and the block finishes within S steps."""
    torch = dev["torch"]
    s = synth.config_step(cfg)
    p = s["params"]
    ds = _ds(dev, s)
    nxt = acceptance.block_loop_logits(p, cfg)
    logits = nxt(s["logits"])
    o_masked, o_tokens = s["masked"].copy(), s["tokens"].copy()   # the oracle's own loop
    steps, diverged_at = 0, None
    total = dict(margin=0, rank=0, tau=0, excluded=0)
    while True:
        torch.cuda.synchronize()
        gm, gt = ds.masked.cpu().numpy().copy(), ds.tokens.cpu().numpy().copy()
        if gm.sum() == 0:
            break
        steps += 1
        _say("cfg%d step %d masked=%d" % (cfg, steps, int(gm.sum())))
        assert steps <= p["S"], "block not finished within S steps"
        if diverged_at is None:
            np.testing.assert_array_equal(gm, o_masked)
            np.testing.assert_array_equal(gt, o_tokens)
        ds.confidence_commit(logits=torch.from_numpy(np.ascontiguousarray(logits)).cuda())
        c, ref = _compare_commit(dev, ds, p, gm, gt, logits, "cfg%d step%d" % (cfg, steps))
        for key in total:
            total[key] += c[key]
        torch.cuda.synchronize()
        nm, nt = ds.masked.cpu().numpy(), ds.tokens.cpu().numpy()
        for r in range(p["n_req"]):
            kept = gm[r] == 0
            np.testing.assert_array_equal(nt[r][kept], gt[r][kept])     # committed tokens stay
            assert np.all(nm[r][kept] == 0)                              # never re-masked
            k = oracle.commit_k(p["D"], p["S"], int(gm[r].sum()))
            assert int(gm[r].sum()) - int(nm[r].sum()) >= k
        if diverged_at is None:
            o_masked, o_tokens = ref["masked"], ref["tokens"]
            if not (np.array_equal(nm, o_masked) and np.array_equal(nt, o_tokens)):
                diverged_at = steps   # only possible at an excluded (counted) position
                _say("cfg%d: trajectory left the oracle's at step %d through a fragile decision" % (cfg, steps))
        logits = nxt(None)
    _say("cfg%d finished in %d steps; fragile %s" % (cfg, steps, total))
    if diverged_at is None:
        want = FRAGILE_COUNTS[str(cfg)]["block_loop"]
        assert steps == want["steps"]
        assert total == {k: want[k] for k in ("margin", "rank", "tau", "excluded")}
    else:
        assert total["excluded"] > 0


def test_commit_last_step_with_slot0_committed(dev):
    """The last step of a block whose slot 0 is already committed and whose every
    remaining masked slot commits now (|M| <= k): every output is written by the
    finishing workgroup, after all workgroups of the launch have read the masked
    flags that it rewrites."""
    torch = dev["torch"]
    p = synth.params_for(1, n_items=1, n_req=3, D=16, n_masked=3, V=151936, S=4, tau=1.5,
                         logit_sigma2=4.0, prefix=("fixed", 8), Hq=2, Hkv=1, d=64, dtype=F32)
    s = synth.make_step(p, seed=616)
    for r, slots in enumerate([[3, 7, 11], [1, 2, 15], [5, 6, 9]]):
        s["masked"][r] = 0
        s["masked"][r, slots] = 1                  # slot 0 committed in every request
        s["tokens"][r] = np.where(s["masked"][r] == 1, -1, 1000 + r)
    ds = _ds(dev, s)
    for rep in range(3):
        ds.reset_block_state()
        ds.conf.fill_(0.5)
        ds.argmax.fill_(7)
        ds.committed.fill_(9)
        ds.n_committed.fill_(9)
        ds.confidence_commit()
        _compare_commit(dev, ds, p, s["masked"], s["tokens"], s["logits"], "last_step_%d" % rep)
        torch.cuda.synchronize()
        assert ds.n_committed.cpu().numpy().tolist() == [3, 3, 3]
        assert int(ds.masked.sum()) == 0
        assert np.array_equal(ds.committed.cpu().numpy(), s["masked"])


COMMIT_CASES = [
    ("none_masked", dict(n_masked=0)),
    ("one_masked", dict(n_masked=1)),
    ("D64_k", dict(D=64, n_masked=50, S=5)),
    ("tau_ge_1", dict(tau=1.0)),
    ("tau_low", dict(tau=0.01)),
    ("V_odd", dict(V=1001)),
    ("V_small", dict(V=2)),
    ("many_req", dict(n_req=12, n_items=1, D=8, n_masked=5, V=5000)),
]


@pytest.mark.parametrize("label,ov", COMMIT_CASES, ids=[c[0] for c in COMMIT_CASES])
def test_confidence_commit_edge_cases(dev, label, ov):
    base = dict(n_items=1, n_req=3, D=16, n_masked=9, V=20000, S=4, tau=0.05, logit_sigma2=1.0,
                prefix=("fixed", 8), Hq=2, Hkv=1, d=64, dtype=F32)
    base.update(ov)
    p = synth.params_for(1, **base)
    s = synth.make_step(p, seed=len(label) * 31)
    _say("confidence_commit %s" % label)
    ds = _ds(dev, s)
    ds.confidence_commit()
    _compare_commit(dev, ds, p, s["masked"], s["tokens"], s["logits"], label)


def test_confidence_ties_and_equal_rows(dev):
    """Exact ties: equal logits give conf 1/V and token 0; equal confidences rank by index."""
    torch = dev["torch"]
    p = synth.params_for(1, n_req=1, D=6, n_masked=6, V=4096, S=3, tau=2.0, prefix=("fixed", 8),
                         Hq=2, Hkv=1, d=64, dtype=F32)
    s = synth.make_step(p, seed=5)
    s["logits"][:] = 0.25
    s["logits"][0, 4, [100, 7, 4000]] = 3.0
    ds = _ds(dev, s)
    ds.confidence_commit()
    torch.cuda.synchronize()
    conf = ds.conf.cpu().numpy()[0]
    arg = ds.argmax.cpu().numpy()[0]
    assert arg.tolist() == [0, 0, 0, 0, 7, 0]
    assert abs(conf[0] - 1.0 / 4096) < 1e-9
    assert ds.committed.cpu().numpy()[0].tolist() == [1, 0, 0, 0, 1, 0]   # k = 2: slot 4, then slot 0


# Seeded random sweep of the row kernels' shapes: request count, block length,
# vocabulary (odd sizes and sizes at 1024-multiples included), masked count,
# S, tau and logit scale drawn together; a quarter of the cases plant a peak.
N_ROW_SWEEP = 16


def _row_sweep_params(i):
    rng = np.random.default_rng(7000 + i)
    while True:
        n_req = int(rng.integers(1, 9))
        D = int(rng.choice([1, 2, 7, 8, 16, 31, 32, 64]))
        V = int(rng.choice([2, int(rng.integers(3, 5000)), 1024 * int(rng.integers(1, 160)) + int(rng.integers(-1, 2)),
                            int(rng.integers(5000, 160000))], p=[0.1, 0.3, 0.3, 0.3]))
        if n_req * D * V <= 2e7:
            break
    return dict(n_items=1, n_req=n_req, D=D, V=V, n_masked=int(rng.integers(0, D + 1)),
                S=int(rng.integers(1, D + 1)), tau=float(rng.choice([0.01, 0.2, 0.5, 0.9, 1.5])),
                logit_sigma2=float(rng.choice([0.25, 1.0, 4.0, 16.0])), plant="peak8" if rng.random() < 0.25 else None,
                prefix=("fixed", 8), Hq=2, Hkv=1, d=64, dtype=F32)


@pytest.mark.parametrize("i", range(N_ROW_SWEEP))
def test_confidence_commit_random_sweep(dev, i):
    p = synth.params_for(1, **_row_sweep_params(i))
    s = synth.make_step(p, seed=7000 + i)
    label = "commit_sweep%d" % i
    _say("%s n_req=%d D=%d V=%d masked=%d S=%d tau=%g sigma2=%g plant=%s" % (
        label, p["n_req"], p["D"], p["V"], p["n_masked"], p["S"], p["tau"], p["logit_sigma2"], p["plant"]))
    ds = _ds(dev, s)
    ds.confidence_commit()
    _compare_commit(dev, ds, p, s["masked"], s["tokens"], s["logits"], label)


@pytest.mark.parametrize("i", range(N_ROW_SWEEP))
def test_verify_random_sweep(dev, i):
    q = _row_sweep_params(100 + i)
    p = synth.params_for(4, **dict(q, plant="geom0.3", D=min(q["D"], 32)))
    s = synth.make_step(p, seed=7100 + i)
    _say("verify_sweep%d n_req=%d D=%d V=%d planted=%s" % (i, p["n_req"], p["D"], p["V"], s["planted_L"].tolist()))
    ds = _ds(dev, s)
    L = ds.verify()
    dev["torch"].cuda.synchronize()
    L_ref, amax_ref = oracle.spec_verify(s["logits"], s["draft"])
    np.testing.assert_array_equal(L.cpu().numpy(), L_ref)
    np.testing.assert_array_equal(L_ref, s["planted_L"])
    np.testing.assert_array_equal(ds.argmax.cpu().numpy(), amax_ref)


# ---------------------------------------------------------------------------
# Speculative verify and KV append
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", list(range(8)))
def test_verify_then_append_cfg4(dev, seed):
    torch = dev["torch"]
    forced = {0: 0, 1: 16}.get(seed)
    s = synth.make_step(synth.params_for(4), synth.seed_of(4) + seed, plant_L=forced)
    p = s["params"]
    _say("verify+append cfg4 seed=%d planted L=%d" % (seed, int(s["planted_L"][0])))
    ds = _ds(dev, s)
    ds.attn()
    L_gpu = ds.verify()
    ds.append(n_accept=L_gpu)
    torch.cuda.synchronize()
    L_ref, amax_ref = oracle.spec_verify(s["logits"], s["draft"])
    assert int(L_gpu.cpu()[0]) == int(L_ref[0]) == int(s["planted_L"][0])
    np.testing.assert_array_equal(ds.argmax.cpu().numpy(), amax_ref)
    kc, vc, pref, err = oracle.kv_append(s["k_cache"], s["v_cache"], s["prefix"], s["k_blk"], s["v_blk"], L_ref)
    assert err == 0 and int(ds.dev_err.cpu()[0]) == 0
    np.testing.assert_array_equal(ds.prefix.cpu().numpy(), pref)
    assert ds.k_cache.cpu().numpy().view(np.uint16).tobytes() == kc.tobytes()
    assert ds.v_cache.cpu().numpy().view(np.uint16).tobytes() == vc.tobytes()


def test_verify_ragged_requests(dev):
    torch = dev["torch"]
    p = synth.params_for(4, n_req=6, n_items=1, D=13, V=3001, prefix=("fixed", 8))
    s = synth.make_step(p, seed=9)
    ds = _ds(dev, s)
    L = ds.verify()
    torch.cuda.synchronize()
    L_ref, amax_ref = oracle.spec_verify(s["logits"], s["draft"])
    np.testing.assert_array_equal(L.cpu().numpy(), L_ref)
    np.testing.assert_array_equal(L_ref, s["planted_L"])
    np.testing.assert_array_equal(ds.argmax.cpu().numpy(), amax_ref)


@pytest.mark.parametrize("cfg", [3, 4, 5])
def test_row_calls_leave_workspace_zeroed(dev, cfg):
    """The confidence / verify kernel publishes its partials into tagged
    workspace slots; the finishing workgroup clears them, and the ticket
    counters, before the call ends.  After every call the whole workspace is
    zero again, and a repeated call on it gives bitwise the same outputs."""
    torch = dev["torch"]
    s = synth.config_step(cfg)
    p = s["params"]
    ds = _ds(dev, s)
    outs = []
    for rep in range(3):
        _say("cfg%d row call %d" % (cfg, rep))
        if cfg == 4:
            L = ds.verify()
            torch.cuda.synchronize()
            assert int(ds.verify_ws.count_nonzero()) == 0
            outs.append([L.cpu().clone(), ds.argmax.cpu().clone()])
        else:
            ds.reset_block_state()
            ds.confidence_commit()
            torch.cuda.synchronize()
            assert int(ds.commit_ws.count_nonzero()) == 0
            outs.append([t.cpu().clone() for t in (ds.conf, ds.argmax, ds.committed, ds.n_committed,
                                                   ds.masked, ds.tokens)])
    for later in outs[1:]:
        for a, b in zip(outs[0], later):
            assert a.numpy().tobytes() == b.numpy().tobytes()  # bitwise (unmasked confidences are NaN)
    if cfg == 4:
        L_ref, amax_ref = oracle.spec_verify(s["logits"], s["draft"])
        np.testing.assert_array_equal(outs[0][0].numpy(), L_ref)
    else:
        _compare_commit(dev, ds, p, s["masked"], s["tokens"], s["logits"], "cfg%d repeated" % cfg)


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_append_overflow_and_partial(dev, dtype):
    torch = dev["torch"]
    p = synth.params_for(1, n_items=3, D=8, dtype=dtype, prefix=("list", [10, 0, 50]), Hq=4, Hkv=2,
                         d=64, cap=64)
    s = synth.make_step(p, seed=3)
    ds = _ds(dev, s)
    acc = np.array([3, 8, 8], np.int32)     # item 2: 50 + 8 > 56? no: cap 64 -> fits
    acc[2] = 8
    s_prefix = s["prefix"].copy()
    s_prefix[2] = 60                        # 60 + 8 > 64: overflow for item 2
    ds.prefix.copy_(torch.from_numpy(s_prefix))
    ds.append(n_accept=torch.from_numpy(acc).cuda())
    torch.cuda.synchronize()
    kc, vc, pref, err = oracle.kv_append(s["k_cache"], s["v_cache"], s_prefix, s["k_blk"], s["v_blk"], acc)
    assert err == 1 and int(ds.dev_err.cpu()[0]) == 1
    np.testing.assert_array_equal(ds.prefix.cpu().numpy(), pref)
    el = np.uint16 if dtype == BF16 else np.float32
    assert ds.k_cache.cpu().numpy().view(el).tobytes() == kc.tobytes()
    assert ds.v_cache.cpu().numpy().view(el).tobytes() == vc.tobytes()


# ---------------------------------------------------------------------------
# LM head fused with confidence + commit (the logits never reach memory).
# The oracle forms fp64 logits, rounds them to fp32 and applies its confidence /
# commit; the GPU sums bf16 products in fp32 (MFMA).  Its logits therefore
# differ from the exact ones by ~1e-5, so a slot whose two largest exact logits
# are within LOGIT_GAP has a fragile greedy token: it is excluded from the
# token comparison (and counted) like a fragile commit decision.
# ---------------------------------------------------------------------------

LOGIT_GAP = 1e-3


class _LmDev:
    def __init__(self, dev, st):
        torch = dev["torch"]
        bd = dev["bd"]
        p = st["params"]
        self.p = p
        c = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        g = _guarded(dev)
        poison = dev["step"].POISON
        self.hidden = c(st["hidden"].view(np.int16))
        self.weight = c(st["weight"].view(np.int16))
        self.masked = g.make("masked", st["masked"].shape, torch.uint8, init=c(st["masked"]))
        self.tokens = g.make("tokens", st["tokens"].shape, torch.int32, init=c(st["tokens"]))
        nr, D = p["n_req"], p["D"]
        self.conf = g.make("conf", (nr, D), torch.float32, fill=poison)
        self.argmax = g.make("argmax", (nr, D), torch.int32, fill=poison)
        self.committed = g.make("committed", (nr, D), torch.uint8, fill=poison)
        self.n_committed = g.make("n_committed", (nr,), torch.int32, fill=poison)
        self.desc = bd.lmhead_desc(nr, D, p["V"], p["H"], p["S"], p["tau"])
        need = bd.bd_lmhead_workspace_bytes(self.desc)
        assert need < bd.SIZE_MAX
        self.ws = g.make("ws", (max(need, 16),), torch.uint8, fill=0)
        self.bd = bd

    def run(self):
        self.bd.bd_lmhead_confidence_commit(self.desc, self.hidden, self.weight, self.masked, self.tokens,
                                            self.conf, self.argmax, self.committed, self.n_committed, self.ws)


def _compare_lmhead(dev, g, st, label):
    torch = dev["torch"]
    torch.cuda.synchronize()
    p = st["params"]
    logits64 = oracle.lm_head_logits(st["hidden"], st["weight"])
    logits32 = logits64.astype(np.float32)
    ref = oracle.confidence_commit(logits32, st["masked"], st["tokens"], p["S"], p["tau"])
    frag_sets = acceptance.step_fragility(logits32, st["masked"], p["S"], p["tau"], ref)
    g_conf, g_arg = g.conf.cpu().numpy(), g.argmax.cpu().numpy()
    g_com, g_ncom = g.committed.cpu().numpy(), g.n_committed.cpu().numpy()
    g_mask, g_tok = g.masked.cpu().numpy(), g.tokens.cpu().numpy()
    excluded = 0
    for r in range(p["n_req"]):
        m = st["masked"][r].astype(bool)
        nm = int(m.sum())
        k = min(-(-p["D"] // p["S"]), nm)
        assert np.all(np.isnan(g_conf[r][~m])) and np.all(g_arg[r][~m] == -1)
        frag = frag_sets[r]["rank"] | frag_sets[r]["tau"]
        for i in np.flatnonzero(m):
            top2 = np.partition(logits64[r, i], -2)[-2:]
            if top2[1] - top2[0] < LOGIT_GAP:
                frag.add(int(i))
            else:
                assert g_arg[r, i] == ref["argmax"][r, i], (label, r, i)
            assert abs(float(g_conf[r, i]) - ref["conf"][r, i]) <= CONF_ABS, (label, r, i)
        own = _rule_commit(g_conf[r], m, k, p["tau"])
        assert set(np.nonzero(g_com[r])[0].tolist()) == own, (label, r)
        excluded += len(frag)
        for i in range(p["D"]):
            if i in frag:
                continue
            assert g_com[r, i] == ref["committed"][r, i], (label, r, i)
            assert g_mask[r, i] == ref["masked"][r, i]
            assert g_tok[r, i] == ref["tokens"][r, i]
        assert g_ncom[r] == int(g_com[r].sum())
        np.testing.assert_array_equal(g_tok[r][~m], st["tokens"][r][~m])
    return excluded, ref


@pytest.mark.parametrize("cfg", [1, 2])
def test_lmhead_configs(dev, cfg):
    st = synth.lmhead_step(cfg)
    p = st["params"]
    _say("lmhead cfg%d n_req=%d D=%d V=%d H=%d" % (cfg, p["n_req"], p["D"], p["V"], p["H"]))
    g = _LmDev(dev, st)
    g.run()
    excl, ref = _compare_lmhead(dev, g, st, "lmhead cfg%d" % cfg)
    # the planted slots are confident and committed
    for r, i, v_star in st["planted"]:
        assert ref["argmax"][r, i] == v_star and ref["committed"][r, i] == 1
    _say("lmhead cfg%d excluded fragile decisions: %d" % (cfg, excl))


LMHEAD_CASES = [
    ("V2", dict(V=2)),
    ("V17_one_tile_plus_one", dict(V=17)),
    ("D1", dict(n_req=1, D=1, n_masked=1, plants=0)),
    ("sixteen_requests", dict(n_req=16, D=1, n_masked=1, plants=1)),
    ("H4096_lds_over_64k", dict(H=4096, V=3001)),
    ("H3584_7B_hidden", dict(H=3584, V=4099, n_req=1, D=16, n_masked=16, S=8, tau=0.8)),
    ("none_masked", dict(n_masked=0, plants=0)),
    ("tau_ge_1", dict(tau=1.0)),
    ("many_tiles", dict(V=65537, n_req=1, D=16, n_masked=12, S=3)),
]


@pytest.mark.parametrize("label,ov", LMHEAD_CASES, ids=[c[0] for c in LMHEAD_CASES])
def test_lmhead_edge_cases(dev, label, ov):
    p = dict(synth.LMHEAD_CONFIGS[2])
    p.update(ov)
    st = synth.make_lmhead(p, seed=len(label) * 17 + 5)
    _say("lmhead %s n_req=%d D=%d V=%d H=%d" % (label, p["n_req"], p["D"], p["V"], p["H"]))
    g = _LmDev(dev, st)
    g.run()
    _compare_lmhead(dev, g, st, label)


# Seeded random sweep of LM-head shapes: hidden size (multiples of 256 up to
# 4096), vocabulary (tiny, odd, and past several 16-row tiles), requests,
# block length, masked count, S, tau and the number of planted peaks.
N_LMHEAD_SWEEP = 8


def _lmhead_sweep_case(i):
    rng = np.random.default_rng(8000 + i)
    while True:
        H = 256 * int(rng.integers(1, 17))
        V = int(rng.choice([int(rng.integers(2, 40)), int(rng.integers(40, 5000)), int(rng.integers(5000, 40000))]))
        D = int(rng.choice([1, 4, 8, 16]))
        n_req = int(rng.integers(1, 16 // D + 1))  # at most 16 slots per call
        if n_req * D * H * V <= 4e8:  # keeps the fp64 oracle within seconds
            break
    n_masked = int(rng.integers(0, D + 1))
    p = dict(synth.LMHEAD_CONFIGS[2], H=H, V=V, n_req=n_req, D=D, n_masked=n_masked, S=int(rng.integers(1, D + 1)),
             tau=float(rng.choice([0.05, 0.5, 0.9, 1.2])), plants=int(rng.integers(0, n_masked + 1)))
    return synth.make_lmhead(p, seed=8000 + i)


@pytest.mark.parametrize("i", range(N_LMHEAD_SWEEP))
def test_lmhead_random_sweep(dev, i):
    st = _lmhead_sweep_case(i)
    p = st["params"]
    label = "lmhead_sweep%d" % i
    _say("%s n_req=%d D=%d V=%d H=%d masked=%d S=%d tau=%g plants=%d" % (
        label, p["n_req"], p["D"], p["V"], p["H"], p["n_masked"], p["S"], p["tau"], p["plants"]))
    g = _LmDev(dev, st)
    g.run()
    _compare_lmhead(dev, g, st, label)


def test_lmhead_deterministic_and_reusable_workspace(dev):
    torch = dev["torch"]
    st = synth.lmhead_step(2)
    g = _LmDev(dev, st)
    outs = []
    for _ in range(3):
        g.masked.copy_(torch.from_numpy(st["masked"]))
        g.tokens.copy_(torch.from_numpy(st["tokens"]))
        g.run()
        torch.cuda.synchronize()
        outs.append((g.conf.cpu().numpy().copy(), g.argmax.cpu().numpy().copy(), g.committed.cpu().numpy().copy()))
    for o in outs[1:]:
        np.testing.assert_array_equal(np.nan_to_num(o[0], nan=-1), np.nan_to_num(outs[0][0], nan=-1))
        np.testing.assert_array_equal(o[1], outs[0][1])
        np.testing.assert_array_equal(o[2], outs[0][2])
