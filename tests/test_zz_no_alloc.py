"""bd_attn_step_noalloc: bd_attn_step with its split-K exchange in the library's
fixed device scratch (for callers that cannot allocate).  On the GPU its output
must equal bd_attn_step's bit for bit, and the oracle's within the bf16 bar, on
two calls in a row, the second with a smaller input; on the host, a call needing
more than the fixed scratch is refused before anything is launched."""

import ctypes
import sys

import numpy as np
import pytest

import oracle
import synth
from synth import BF16, BIDIR, CAUSAL, F32

ATTN_MAX_ABS = 2e-2
ATTN_REL = 1e-2


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_noalloc_refuses_calls_beyond_its_scratch():
    from vlm_decoding_amd import bd
    limit = bd.lib.bd_attn_noalloc_max_scratch_bytes()
    assert limit == 64 << 20
    fake = 1 << 20
    # 64 items of a quadratic block of 32 drafts (560 slots) at prefix 8192
    big = bd.attn_desc(64, 32, 16, 2, 128, 8192 + 560, BF16, bd.BD_BLOCK_QUAD, 8192)
    need = bd.bd_attn_workspace_bytes(big)
    assert limit < need < bd.SIZE_MAX
    st = bd.lib.bd_attn_step_noalloc(ctypes.byref(big), fake, fake, fake, fake, fake, fake, fake, None)
    assert st == bd.BD_E_SCRATCH
    assert b"scratch" in bd.lib.bd_status_string(st)
    # validation still comes first
    bad = bd.attn_desc(1, 8, 16, 2, 96, 1024, BF16, BIDIR, 512)
    assert bd.lib.bd_attn_step_noalloc(ctypes.byref(bad), fake, fake, fake, fake, fake, fake, fake, None) == bd.BD_E_SHAPE
    ok = bd.attn_desc(1, 8, 16, 2, 128, 1024, BF16, BIDIR, 512)
    assert bd.lib.bd_attn_step_noalloc(ctypes.byref(ok), None, fake, fake, fake, fake, fake, fake, None) == bd.BD_E_NULL


def _check(got, ref, label):
    err = np.abs(got - ref)
    rel = max(float(np.linalg.norm((got[i] - ref[i]).ravel()) / np.linalg.norm(ref[i].ravel()))
              for i in range(ref.shape[0]))
    _say("%s: max_abs=%.3g max_rel_l2=%.3g" % (label, float(err.max()), rel))
    assert np.all(np.isfinite(got)) and float(err.max()) <= ATTN_MAX_ABS and rel <= ATTN_REL, label


CASES = [
    # (label, overrides, mode, items checked against the oracle)
    # the headline shape with ragged prefixes: more split slots than CUs, so the
    # tile kernel runs paired halves (some slots absorbed, some units written out)
    ("36_layers_paired_ragged", dict(n_items=36, prefix=("list", [4096 - 117 * i for i in range(36)])), BIDIR, [0, 35]),
    ("8_layers_prefix_4096", dict(n_items=8, prefix=("fixed", 4096)), BIDIR, [0, 7]),
    ("2_items_ragged_smaller", dict(n_items=2, prefix=("list", [700, 33])), CAUSAL, [0, 1]),
    # the balanced split plan (a mode flag): its exchange also holds each unit's split count
    ("4_items_ragged_balanced", dict(n_items=4, prefix=("list", [3000, 150, 1700, 4096])), BIDIR, [1, 3]),
]


@pytest.mark.gpu
def test_noalloc_matches_bd_attn_step_on_two_calls_in_a_row():
    import torch
    from vlm_decoding_amd import bd
    from vlm_decoding_amd.step import DeviceStep
    assert torch.cuda.is_available()
    for label, ov, mode, items in CASES:
        p = synth.params_for(3, dtype=BF16, D=16, n_masked=8, V=1000, plant=None, mode=mode, **ov)
        st = synth.make_step(p, seed=len(label) * 101)
        _say("noalloc %s n=%d mode=%d prefix=%s" % (label, p["n_items"], mode, st["prefix"].tolist()))
        ds = DeviceStep(st, balanced=label.endswith("balanced"))
        ds.attn()
        torch.cuda.synchronize()
        want = ds.out.clone()
        ds.out.fill_(0x5A5A)
        bd.bd_attn_step_noalloc(ds.adesc, ds.q, ds.k_blk, ds.v_blk, ds.k_cache, ds.v_cache, ds.prefix, ds.out)
        torch.cuda.synchronize()
        assert torch.equal(ds.out, want), label
        got = synth.bf16_bits_to_f32(ds.out.cpu().numpy().view(np.uint16)).astype(np.float64)[items]
        sl = lambda a: np.ascontiguousarray(a[items])
        ref = oracle.attention(*[sl(st[k]) for k in ("q", "k_blk", "v_blk", "k_cache", "v_cache", "prefix")], mode)
        _check(got, ref, "noalloc_" + label)


@pytest.mark.gpu
def test_noalloc_fp32_path_uses_no_scratch():
    import torch
    from vlm_decoding_amd import bd
    from vlm_decoding_amd.step import DeviceStep
    p = synth.params_for(1, n_items=3, prefix=("list", [0, 70, 129]), Hq=6, Hkv=2, D=5, dtype=F32)
    st = synth.make_step(p, seed=77)
    ds = DeviceStep(st)
    ds.attn()
    torch.cuda.synchronize()
    want = ds.out.clone()
    ds.out.zero_()
    bd.bd_attn_step_noalloc(ds.adesc, ds.q, ds.k_blk, ds.v_blk, ds.k_cache, ds.v_cache, ds.prefix, ds.out)
    torch.cuda.synchronize()
    assert torch.equal(ds.out, want)
