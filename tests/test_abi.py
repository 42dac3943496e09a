"""The C ABI on the host: every symbol that include/bd.h declares is exported by
libbd.so, and argument validation rejects bad calls before anything is launched
(no GPU needed: validation returns before the first HIP call)."""

import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bd.h")


@pytest.fixture(scope="module")
def bd():
    from vlm_decoding_amd import bd as mod
    return mod


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(bd_[a-z0-9_]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for must in ["bd_attn_step", "bd_attn_step_fp8kv", "bd_confidence_commit", "bd_spec_verify", "bd_kv_append",
                 "bd_lmhead_confidence_commit", "bd_two_stream_attn"]:
        assert must in names
    assert len(names) >= 12


def test_library_exports_every_declared_symbol(bd):
    lib = ctypes.CDLL(bd.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def _attn(bd, **kw):
    base = dict(n_items=36, D=16, Hq=16, Hkv=2, d=128, cap=4160, dtype=1, mode=0, max_prefix=4096, scale=0.0884)
    base.update(kw)
    return bd.BdAttnDesc(*[base[f] for f, _ in bd.BdAttnDesc._fields_])


BAD_ATTN = [
    (dict(d=96), "BD_E_SHAPE"), (dict(D=0), "BD_E_SHAPE"), (dict(D=65), "BD_E_SHAPE"),
    (dict(Hq=15), "BD_E_SHAPE"), (dict(Hkv=0), "BD_E_SHAPE"), (dict(cap=0), "BD_E_SHAPE"),
    (dict(max_prefix=5000), "BD_E_SHAPE"), (dict(max_prefix=-1), "BD_E_SHAPE"), (dict(n_items=0), "BD_E_SHAPE"),
    (dict(dtype=7), "BD_E_DTYPE"), (dict(mode=3), "BD_E_PARAM"), (dict(scale=float("nan")), "BD_E_PARAM"),
    (dict(scale=0.0), "BD_E_PARAM"), (dict(scale=float("inf")), "BD_E_PARAM"),
    # launches past 32-bit grids: 2^27 items x 2 KV heads x 64 splits; 2^29 items x 64 slots x 128 heads
    (dict(n_items=1 << 27), "BD_E_SHAPE"), (dict(n_items=(1 << 29) - 1, D=64, Hq=128, Hkv=128, max_prefix=0), "BD_E_SHAPE"),
]


@pytest.mark.parametrize("kw,code", BAD_ATTN)
def test_attn_validation(bd, kw, code):
    desc = _attn(bd, **kw)
    fake = 1 << 20  # never dereferenced: validation fails first
    st = bd.lib.bd_attn_step(ctypes.byref(desc), fake, fake, fake, fake, fake, fake, fake, fake, 1 << 30, None)
    assert st == getattr(bd, code)
    assert bd.lib.bd_attn_workspace_bytes(ctypes.byref(desc)) == bd.SIZE_MAX


@pytest.mark.parametrize("dtype", [0, 1, 2])
def test_any_cache_capacity_is_accepted(bd, dtype):
    """K and V caches are both [cap][d] rows of d * element-size bytes (a multiple of
    16), so no capacity needs rounding: odd and small ones are valid shapes."""
    for cap in (4096, 4097, 4099, 4103):
        assert bd.lib.bd_attn_workspace_bytes(ctypes.byref(_attn(bd, cap=cap, dtype=dtype))) != bd.SIZE_MAX
    assert bd.lib.bd_attn_workspace_bytes(ctypes.byref(_attn(bd, cap=1, max_prefix=1, dtype=dtype))) != bd.SIZE_MAX


def test_balanced_plan_flag(bd):
    """BD_PLAN_BALANCED is a flag on the mode: accepted with every mask mode, other
    high bits refused; with it a ragged batch of up to 64 items may use more
    split slots per unit (a larger workspace), never fewer."""
    fake = 1 << 20
    for mode in (0, 1, 2):
        plain = _attn(bd, n_items=8, mode=mode, D=8 if mode == 2 else 16)
        flagged = _attn(bd, n_items=8, mode=mode | bd.BD_PLAN_BALANCED, D=8 if mode == 2 else 16)
        a, b = bd.bd_attn_workspace_bytes(plain), bd.bd_attn_workspace_bytes(flagged)
        assert a < bd.SIZE_MAX and a <= b < bd.SIZE_MAX, (mode, a, b)
    for bad in (0x200, bd.BD_PLAN_BALANCED | 3, 0x101 | 0x400):
        desc = _attn(bd, mode=bad)
        assert bd.bd_attn_workspace_bytes(desc) == bd.SIZE_MAX
        st = bd.lib.bd_attn_step(ctypes.byref(desc), fake, fake, fake, fake, fake, fake, fake, fake, 1 << 30, None)
        assert st == bd.BD_E_PARAM
    # the append reads the flagged descriptor's mask mode
    desc = _attn(bd, mode=bd.BD_BLOCK_QUAD | bd.BD_PLAN_BALANCED, D=33)
    assert bd.lib.bd_kv_append(ctypes.byref(desc), fake, fake, fake, fake, fake, None, None, None) == bd.BD_E_SHAPE
    # beyond 64 items the flag is ignored: the plain plan's workspace
    big_plain, big_flag = _attn(bd, n_items=65), _attn(bd, n_items=65, mode=bd.BD_PLAN_BALANCED)
    assert bd.bd_attn_workspace_bytes(big_plain) == bd.bd_attn_workspace_bytes(big_flag)


def test_attn_null_and_workspace_errors(bd):
    desc = _attn(bd)
    fake = 1 << 20
    assert bd.lib.bd_attn_step(None, fake, fake, fake, fake, fake, fake, fake, fake, 1 << 30, None) == bd.BD_E_NULL
    assert bd.lib.bd_attn_step(ctypes.byref(desc), None, fake, fake, fake, fake, fake, fake, fake, 1 << 30, None) == bd.BD_E_NULL
    need = bd.lib.bd_attn_workspace_bytes(ctypes.byref(desc))
    assert 0 < need < bd.SIZE_MAX
    assert bd.lib.bd_attn_step(ctypes.byref(desc), fake, fake, fake, fake, fake, fake, fake, fake, need - 1, None) == bd.BD_E_WORKSPACE
    assert bd.lib.bd_attn_step(ctypes.byref(desc), fake, fake, fake, fake, fake, fake, fake, None, need, None) == bd.BD_E_WORKSPACE
    assert bd.lib.bd_attn_step(ctypes.byref(desc), fake + 2, fake, fake, fake, fake, fake, fake, fake, need, None) == bd.BD_E_PARAM


def test_single_split_needs_no_workspace(bd):
    # A prefix shorter than one 32-key tile never splits.
    for mp in (0, 16, 31):
        desc = _attn(bd, n_items=1, max_prefix=mp, cap=128)
        assert bd.lib.bd_attn_workspace_bytes(ctypes.byref(desc)) == 0
    desc32 = _attn(bd, dtype=0)
    assert bd.lib.bd_attn_workspace_bytes(ctypes.byref(desc32)) == 0


def _fp8_call(bd, desc, k_scale=1 << 20, v_scale=1 << 20, ws_bytes=1 << 30, q=1 << 20, ws=1 << 20):
    fake = 1 << 20
    return bd.lib.bd_attn_step_fp8kv(ctypes.byref(desc) if desc is not None else None, q, fake, fake, fake, fake,
                                     k_scale, v_scale, fake, fake, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", BAD_ATTN)
def test_fp8kv_attn_validation(bd, kw, code):
    # The shape rules of bd_attn_step.
    desc = _attn(bd, **dict(dict(dtype=bd.BD_FP8KV), **kw))
    assert _fp8_call(bd, desc) == getattr(bd, code)
    assert bd.lib.bd_attn_workspace_bytes(ctypes.byref(desc)) == bd.SIZE_MAX


def test_fp8kv_dtype_routing_and_errors(bd):
    fake = 1 << 20
    fp8 = _attn(bd, dtype=bd.BD_FP8KV)
    bf16 = _attn(bd, dtype=bd.BD_BF16)
    # Each entry point takes only its own dtype.
    assert _fp8_call(bd, bf16) == bd.BD_E_DTYPE
    assert bd.lib.bd_attn_step(ctypes.byref(fp8), fake, fake, fake, fake, fake, fake, fake, fake, 1 << 30, None) == bd.BD_E_DTYPE
    assert _fp8_call(bd, None) == bd.BD_E_NULL
    assert _fp8_call(bd, fp8, k_scale=None) == bd.BD_E_NULL
    assert _fp8_call(bd, fp8, v_scale=None) == bd.BD_E_NULL
    need = bd.lib.bd_attn_workspace_bytes(ctypes.byref(fp8))
    assert 0 < need < bd.SIZE_MAX
    assert _fp8_call(bd, fp8, ws_bytes=need - 1) == bd.BD_E_WORKSPACE
    assert _fp8_call(bd, fp8, ws=None, ws_bytes=need) == bd.BD_E_WORKSPACE
    assert _fp8_call(bd, fp8, q=fake + 2, ws_bytes=need) == bd.BD_E_PARAM
    # 64-key E4M3 tiles: a prefix below 64 never splits.
    for mp in (0, 32, 63):
        desc = _attn(bd, n_items=1, max_prefix=mp, cap=128, dtype=bd.BD_FP8KV)
        assert bd.lib.bd_attn_workspace_bytes(ctypes.byref(desc)) == 0
    # kv_append copies E4M3 bytes; any capacity is a valid shape (a NULL prefix
    # pointer is what it then refuses).
    assert bd.lib.bd_kv_append(ctypes.byref(_attn(bd, dtype=bd.BD_FP8KV, cap=4169)), fake, fake, None, fake, fake,
                               None, None, None) == bd.BD_E_NULL


def test_quad_mode_validation(bd):
    """Quadratic mode: D is the draft block size B (1..32); its block holds B (B + 3) / 2 slots."""
    fake = 1 << 20
    for B, code in ((0, "BD_E_SHAPE"), (33, "BD_E_SHAPE")):
        desc = _attn(bd, mode=bd.BD_BLOCK_QUAD, D=B)
        assert bd.lib.bd_attn_step(ctypes.byref(desc), fake, fake, fake, fake, fake, fake, fake, fake, 1 << 30,
                                   None) == getattr(bd, code)
        assert bd.lib.bd_attn_workspace_bytes(ctypes.byref(desc)) == bd.SIZE_MAX
    for B in (1, 16, 32):
        desc = _attn(bd, mode=bd.BD_BLOCK_QUAD, D=B)
        assert 0 < bd.lib.bd_attn_workspace_bytes(ctypes.byref(desc)) < bd.SIZE_MAX
    # More slots mean more rows, hence more workspace, than the same B as a plain block.
    quad = bd.lib.bd_attn_workspace_bytes(ctypes.byref(_attn(bd, mode=bd.BD_BLOCK_QUAD, D=16)))
    plain = bd.lib.bd_attn_workspace_bytes(ctypes.byref(_attn(bd, mode=bd.BD_BLOCK_BIDIR, D=16)))
    assert quad > plain
    assert bd.lib.bd_kv_append(ctypes.byref(_attn(bd, mode=3)), fake, fake, fake, fake, fake, None, None,
                               None) == bd.BD_E_PARAM
    assert bd.lib.bd_kv_append(ctypes.byref(_attn(bd, mode=bd.BD_BLOCK_QUAD, D=33)), fake, fake, fake, fake, fake,
                               None, None, None) == bd.BD_E_SHAPE


def _ts(bd, **kw):
    base = dict(n_seq=8, Lc=2048, Ln=832, cap=2880, D=32, Hq=16, Hkv=2, d=128, max_spans=2, scale=0.0884)
    base.update(kw)
    return bd.BdTwoStreamDesc(*[base[f] for f, _ in bd.BdTwoStreamDesc._fields_])


BAD_TWO_STREAM = [
    (dict(n_seq=0), "BD_E_SHAPE"), (dict(Lc=0), "BD_E_SHAPE"), (dict(Ln=-1), "BD_E_SHAPE"), (dict(D=0), "BD_E_SHAPE"),
    (dict(D=4097), "BD_E_SHAPE"), (dict(cap=2848), "BD_E_SHAPE"), (dict(cap=2888), "BD_E_SHAPE"),
    (dict(Hq=15), "BD_E_SHAPE"), (dict(d=96), "BD_E_SHAPE"), (dict(max_spans=0), "BD_E_SHAPE"),
    (dict(max_spans=257), "BD_E_SHAPE"), (dict(scale=float("nan")), "BD_E_PARAM"), (dict(scale=-1.0), "BD_E_PARAM"),
    (dict(n_seq=1 << 24), "BD_E_SHAPE"),  # launch past 32-bit grids
]


@pytest.mark.parametrize("kw,code", BAD_TWO_STREAM)
def test_two_stream_validation(bd, kw, code):
    desc = _ts(bd, **kw)
    fake = 1 << 20
    st = bd.lib.bd_two_stream_attn(ctypes.byref(desc), fake, fake, fake, fake, fake, fake, fake, 1 << 30, None)
    assert st == getattr(bd, code)
    assert bd.lib.bd_two_stream_workspace_bytes(ctypes.byref(desc)) == bd.SIZE_MAX


def test_two_stream_null_alignment_and_workspace(bd):
    fake = 1 << 20
    desc = _ts(bd)
    need = bd.lib.bd_two_stream_workspace_bytes(ctypes.byref(desc))
    assert need < bd.SIZE_MAX
    call = lambda *a: bd.lib.bd_two_stream_attn(ctypes.byref(desc), *a)
    assert bd.lib.bd_two_stream_attn(None, fake, fake, fake, fake, fake, fake, fake, need, None) == bd.BD_E_NULL
    assert call(fake, fake, fake, None, fake, fake, fake, need, None) == bd.BD_E_NULL
    assert call(fake, fake, fake, fake, None, fake, fake, need, None) == bd.BD_E_NULL
    assert call(fake, fake, fake, fake, fake, None, fake, need, None) == bd.BD_E_NULL
    assert call(fake + 2, fake, fake, fake, fake, fake, fake, need, None) == bd.BD_E_PARAM
    if need > 0:
        assert call(fake, fake, fake, fake, fake, fake, fake, need - 1, None) == bd.BD_E_WORKSPACE
    # Without responses (plain causal prefill) the span arrays are not needed.
    plain = _ts(bd, Ln=0, max_spans=0, cap=2048)
    assert bd.lib.bd_two_stream_workspace_bytes(ctypes.byref(plain)) < bd.SIZE_MAX
    # Few, long sequences split their keys (workspace); many sequences fill the GPU without.
    few = _ts(bd, n_seq=1, Hq=2, Hkv=1, Lc=4096, Ln=0, max_spans=0, cap=4096)
    assert bd.lib.bd_two_stream_workspace_bytes(ctypes.byref(few)) > 0


BAD_COMMIT = [
    (dict(n_req=0), "BD_E_SHAPE"), (dict(D=0), "BD_E_SHAPE"), (dict(D=65), "BD_E_SHAPE"), (dict(V=1), "BD_E_SHAPE"),
    (dict(S=0), "BD_E_PARAM"), (dict(tau=float("nan")), "BD_E_PARAM"),
]


@pytest.mark.parametrize("kw,code", BAD_COMMIT)
def test_commit_validation(bd, kw, code):
    base = dict(n_req=1, D=16, V=151936, S=16, tau=0.9)
    base.update(kw)
    desc = bd.BdCommitDesc(base["n_req"], base["D"], base["V"], base["S"], base["tau"])
    fake = 1 << 20
    st = bd.lib.bd_confidence_commit(ctypes.byref(desc), fake, fake, fake, None, None, None, None, fake, 1 << 30, None)
    assert st == getattr(bd, code)
    assert bd.lib.bd_commit_workspace_bytes(ctypes.byref(desc)) == bd.SIZE_MAX


def test_commit_null_and_workspace(bd):
    desc = bd.BdCommitDesc(1, 16, 151936, 16, 0.9)
    fake = 1 << 20
    need = bd.lib.bd_commit_workspace_bytes(ctypes.byref(desc))
    assert 0 < need < bd.SIZE_MAX
    assert bd.lib.bd_confidence_commit(ctypes.byref(desc), None, fake, fake, None, None, None, None, fake, need, None) == bd.BD_E_NULL
    assert bd.lib.bd_confidence_commit(ctypes.byref(desc), fake, fake, fake, None, None, None, None, fake, need - 1, None) == bd.BD_E_WORKSPACE
    # tau >= 1 is legal (the threshold rule is then off); inf too.
    ok = bd.BdCommitDesc(1, 16, 151936, 16, math.inf)
    assert bd.lib.bd_commit_workspace_bytes(ctypes.byref(ok)) == need


def test_verify_and_append_validation(bd):
    fake = 1 << 20
    assert bd.lib.bd_verify_workspace_bytes(1, 0, 100) == bd.SIZE_MAX
    need = bd.lib.bd_verify_workspace_bytes(1, 16, 151936)
    assert bd.lib.bd_spec_verify(1, 16, 151936, fake, None, fake, None, fake, need, None) == bd.BD_E_NULL
    assert bd.lib.bd_spec_verify(1, 16, 151936, fake, fake, fake, None, fake, need - 1, None) == bd.BD_E_WORKSPACE
    assert bd.lib.bd_spec_verify(1, 65, 151936, fake, fake, fake, None, fake, need, None) == bd.BD_E_SHAPE
    desc = _attn(bd, dtype=5)
    assert bd.lib.bd_kv_append(ctypes.byref(desc), fake, fake, fake, fake, fake, None, None, None) == bd.BD_E_DTYPE
    desc = _attn(bd, cap=0)
    assert bd.lib.bd_kv_append(ctypes.byref(desc), fake, fake, fake, fake, fake, None, None, None) == bd.BD_E_SHAPE
    # Rows are copied as 16-byte units: every cache and block pointer must be 16-byte aligned.
    desc = _attn(bd, cap=4099)
    for i in range(4):
        ptrs = [fake] * 4
        ptrs[i] = fake + 8
        kc, vc, kb, vb = ptrs
        assert bd.lib.bd_kv_append(ctypes.byref(desc), kc, vc, fake, kb, vb, None, None, None) == bd.BD_E_PARAM
    desc = _attn(bd)
    assert bd.lib.bd_kv_append(ctypes.byref(desc), None, fake, fake, fake, fake, None, None, None) == bd.BD_E_NULL
    # A block of 64 slots x 2^19 KV heads x d 128 (2^32 elements per item) would
    # overflow 32-bit index arithmetic: refused before any launch.
    desc = _attn(bd, D=64, Hq=1 << 19, Hkv=1 << 19)
    assert bd.lib.bd_kv_append(ctypes.byref(desc), fake, fake, fake, fake, fake, None, None, None) == bd.BD_E_SHAPE
    desc = _attn(bd, D=64, Hq=1 << 16, Hkv=1 << 16)   # 2^29 elements: within the limit
    assert bd.lib.bd_kv_append(ctypes.byref(desc), fake, fake, None, fake, fake, None, None, None) == bd.BD_E_NULL
    desc = _attn(bd, cap=(1 << 23) + 8)               # cap * d > 2^30
    assert bd.lib.bd_kv_append(ctypes.byref(desc), fake, fake, fake, fake, fake, None, None, None) == bd.BD_E_SHAPE


BAD_LMHEAD = [
    (dict(n_req=0), "BD_E_SHAPE"), (dict(D=0), "BD_E_SHAPE"), (dict(D=17), "BD_E_SHAPE"),
    (dict(n_req=2, D=16), "BD_E_SHAPE"), (dict(V=1), "BD_E_SHAPE"), (dict(H=128), "BD_E_SHAPE"),
    (dict(H=2050), "BD_E_SHAPE"), (dict(H=4352), "BD_E_SHAPE"), (dict(S=0), "BD_E_PARAM"),
    (dict(tau=float("nan")), "BD_E_PARAM"),
]


@pytest.mark.parametrize("kw,code", BAD_LMHEAD)
def test_lmhead_validation(bd, kw, code):
    base = dict(n_req=1, D=16, V=151936, H=2048, S=16, tau=0.9)
    base.update(kw)
    desc = bd.BdLmheadDesc(*[base[f] for f, _ in bd.BdLmheadDesc._fields_])
    fake = 1 << 20
    st = bd.lib.bd_lmhead_confidence_commit(ctypes.byref(desc), fake, fake, fake, fake, None, None, None, None,
                                            fake, 1 << 30, None)
    assert st == getattr(bd, code)
    assert bd.lib.bd_lmhead_workspace_bytes(ctypes.byref(desc)) == bd.SIZE_MAX


def test_lmhead_null_alignment_and_workspace(bd):
    desc = bd.BdLmheadDesc(1, 16, 151936, 2048, 16, 0.9)
    fake = 1 << 20
    need = bd.lib.bd_lmhead_workspace_bytes(ctypes.byref(desc))
    assert 0 < need < bd.SIZE_MAX
    call = bd.lib.bd_lmhead_confidence_commit
    assert call(ctypes.byref(desc), None, fake, fake, fake, None, None, None, None, fake, need, None) == bd.BD_E_NULL
    assert call(ctypes.byref(desc), fake, fake, None, fake, None, None, None, None, fake, need, None) == bd.BD_E_NULL
    assert call(ctypes.byref(desc), fake + 8, fake, fake, fake, None, None, None, None, fake, need, None) == bd.BD_E_PARAM
    assert call(ctypes.byref(desc), fake, fake, fake, fake, None, None, None, None, fake, need - 1, None) == bd.BD_E_WORKSPACE
    assert call(ctypes.byref(desc), fake, fake, fake, fake, None, None, None, None, None, need, None) == bd.BD_E_WORKSPACE
    # 7B hidden size (3584) and the largest supported (4096) are accepted
    for H in (3584, 4096):
        ok = bd.BdLmheadDesc(1, 16, 152064, H, 8, 0.8)
        assert bd.lib.bd_lmhead_workspace_bytes(ctypes.byref(ok)) < bd.SIZE_MAX


def test_status_strings(bd):
    for code in range(7):
        assert bd.lib.bd_status_string(code)
    assert bd.lib.bd_status_string(99) == b"unknown status"
    assert bd.lib.bd_last_hip_error() == 0


def test_binding_refuses_to_run_without_the_library(tmp_path):
    """No fallback: the package copied without libbd.so raises on import, for the
    binding and for the step helper built on it."""
    import shutil
    import subprocess
    import sys
    pkg = tmp_path / "vlm_decoding_amd"
    pkg.mkdir()
    for f in ("__init__.py", "bd.py", "step.py"):
        shutil.copy(os.path.join(ROOT, "vlm_decoding_amd", f), str(pkg / f))
    for mod in ("vlm_decoding_amd.bd", "vlm_decoding_amd.step"):
        r = subprocess.run([sys.executable, "-c", "import " + mod], cwd=str(tmp_path), capture_output=True, text=True,
                           env=dict(os.environ, PYTHONPATH=str(tmp_path)), timeout=300)
        assert r.returncode != 0 and "libbd.so is not built" in r.stderr, (mod, r.stderr[-500:])
