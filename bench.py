"""Throughput of one block-diffusion denoise step on one MI355X.

Workload (the long-reasoning 3B-shape step): 36 independent layers of block
attention (16 query / 2 KV heads, head dim 128, bf16, cached prefix 4096,
block D = 16 with 8 slots still masked) in one bd_attn_step call, then one
bd_confidence_commit over the 8 masked rows of a 16 x 151936 fp32 logits
tensor (S = 16, tau = 0.9).  A "step" is exactly those two calls.  The
commit mutates the block state, so each step starts from its own copy of
the initial state (8 of 16 slots masked), prepared before timing.

Inputs are seeded and synthetic.  Four independent input sets (~645 MB) are
rotated so that no step finds its K/V in the 256 MB last-level cache: every
step streams its bytes from HBM.

Prints one JSON line.  ``value`` is timed steps over the wall time of the K
timed steps (bracketed by device synchronisations; one event pair around
them gives the GPU time, ``gpu_event_us_per_step``).  After the timed region
a sampled pass runs the same step max(20, --event-samples) more times with
HIP events on the launch stream around the attention call and the commit
call of every step; ``roofline.achieved`` is the attention call's
algorithmic bytes over the mean of those samples, and median / p10 / p90
are reported with them (``steps_per_s_at_median`` = 1 / the step median).
The events are recorded without the system-scope cache release of a default
event record (hipEventDisableSystemFence), which would cost the GPU several
microseconds per record.

Beside the headline (extra keys): the same step timed cold, one step after
each untimed 1 GiB flush read (``cold_step``); the other configurations of
the workload table (``configs``: the 3B single layer, the 3B verify chain -
causal attention, speculative verify, KV append of the accepted prefix - and
the 7B batch of 8 ragged requests); the layer-serial form of the headline
step in a HIP graph; the next rows of the path (LM head + confidence, E4M3
KV cache, quadratic speculative step, two-stream training attention); and
``cpu_baseline``, the fp64 CPU oracle on this host, one thread and all.
"""

import argparse
import ctypes
import gc
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

CFG = 3
N_SETS = 4
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA, MI355X
FLUSH_BYTES = 1 << 30
METRIC = "denoise steps/sec + achieved HBM GB/s (%peak), 3B-shape block-16, 1 GPU"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "cfg3_step_traffic.json")
HEADLINE_KERNELS = ("attn_mfma_kernel<128, 4, false, false, true>", "attn_merge_kernel<128, 4, 32, false, 4, 16, 1, true>")
FP8KV_KERNELS = ("attn_mfma_kernel<128, 4, true, false, true>", "attn_merge_kernel<128, 4, 64, false, 4, 16, 1, true>")
ROW_KERNEL = "row_kernel<false>"
ATTN_SOURCES = ["vlm_decoding_amd/csrc/bd_attn.hip", "vlm_decoding_amd/csrc/bd_common.h",
                "vlm_decoding_amd/csrc/bd_internal.h"]
ROW_SOURCES = ["vlm_decoding_amd/csrc/bd_rows.hip", "vlm_decoding_amd/csrc/bd_rowreduce.h",
               "vlm_decoding_amd/csrc/bd_common.h", "vlm_decoding_amd/csrc/bd_internal.h"]


# ---------------------------------------------------------------------------
# Timing helpers
# ---------------------------------------------------------------------------

class HipEvents:
    """A pool of HIP events, made through the HIP runtime torch loaded, recorded on
    the launch stream without the system-scope release of a default record."""

    DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so.7")  # the copy torch already loaded
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventQuery.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.ev.append(e)

    def record(self, i, stream_handle):
        if self.hip.hipEventRecord(self.ev[i], ctypes.c_void_p(stream_handle)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def wait(self, i):
        """Poll event i until it has completed (hipErrorNotReady = 600 until then)."""
        while True:
            st = self.hip.hipEventQuery(self.ev[i])
            if st == 0:
                return
            if st != 600:
                raise RuntimeError("hipEventQuery failed (%d)" % st)

    def ms(self, i, j):
        f = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(f), self.ev[i], self.ev[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return f.value

    def destroy(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)
        self.ev = []


def dist_us(ms_list):
    """Median, p10, p90 and mean (microseconds) of event samples in milliseconds."""
    a = np.asarray(ms_list, dtype=np.float64) * 1e3
    return dict(median=round(float(np.median(a)), 2), p10=round(float(np.percentile(a, 10)), 2),
                p90=round(float(np.percentile(a, 90)), 2), mean=round(float(a.mean()), 2), samples=int(a.size))


def timed_calls(torch, stream, calls, iters, flush=None, before=None, sets=1, per_call=False):
    """Time ``iters`` iterations of ``calls(i)`` (a list of C-ABI calls issued on
    ``stream``), each bracketed by HIP events.  ``flush`` (a 1 GiB tensor) is read
    in full before every iteration outside the events, so none of the data the
    iteration touches is left in the L2s or the 256 MB last-level cache (a read,
    not a write: a written flush would leave that cache full of dirty lines for
    the timed iteration to write back); ``before(i)`` runs untimed work (state
    restores) after it.  Returns the per-iteration event times in ms; with
    ``per_call`` an event also follows every call, and the result is one list of
    times per call instead."""
    n_calls = len(calls(0)) if per_call else 1
    ev = HipEvents((n_calls + 1) * iters)
    sh = stream.cuda_stream
    status = 0
    for i in range(iters):
        if flush is not None:
            torch.sum(flush)
        if before is not None:
            before(i)
        e0 = (n_calls + 1) * i
        ev.record(e0, sh)
        for k, (fn, args) in enumerate(calls(i)):
            status |= fn(*args)
            if per_call:
                ev.record(e0 + 1 + k, sh)
        if not per_call:
            ev.record(e0 + 1, sh)
    torch.cuda.synchronize()
    if status:
        ev.destroy()
        raise RuntimeError("a library call failed (status %d)" % status)
    if per_call:
        out = [[ev.ms((n_calls + 1) * i + k, (n_calls + 1) * i + k + 1) for i in range(iters)] for k in range(n_calls)]
    else:
        out = [ev.ms(2 * i, 2 * i + 1) for i in range(iters)]
    ev.destroy()
    return out


# ---------------------------------------------------------------------------
# Algorithmic bytes
# ---------------------------------------------------------------------------

def attn_bytes(p, prefix, kv_elem=2):
    """Bytes a block-attention call must move at least once: every K/V element of
    the prefix and of the block once per KV head, Q read, O written (bf16)."""
    n, D, Hq, Hkv, d = p["n_items"], p["D"], p["Hq"], p["Hkv"], p["d"]
    kv = int(np.sum(prefix.astype(np.int64) + D)) * Hkv * d * kv_elem * 2
    qo = n * D * Hq * d * 2 * 2
    return kv + qo


def commit_bytes(p, n_masked):
    """The masked rows' logits, plus the block state read and written."""
    D, n_req = p["D"], p["n_req"]
    state = n_req * (D * (1 + 4) * 2 + D * (4 + 4 + 1) + 4)  # masked/tokens in+out, conf/argmax/committed, count
    return n_masked * p["V"] * 4, state


def source_hash(paths):
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def committed_traffic():
    """Counter-derived HBM bytes per launch from the committed counter runs, for
    the kernels whose sources have not changed since; else None per kernel."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return {}
    out = {}
    if t.get("attn_source_sha256") == source_hash(ATTN_SOURCES):
        out["attn"] = t.get("attn_bytes_per_launch")
        out["fp8kv"] = t.get("fp8kv_bytes_per_launch")
    if t.get("row_source_sha256") == source_hash(ROW_SOURCES):
        out["commit"] = t.get("commit_bytes_per_launch")
    return out


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on the host
# ---------------------------------------------------------------------------

def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(step, budget_s):
    """The fp64 oracle on the host cores.  All threads: whole headline steps
    (36-layer attention, then confidence + commit) until about budget_s / 2 has
    passed.  One thread: a bounded sample - the attention of 2 of the 36 layers
    (same prefix and block, so each layer costs the same) and the whole
    confidence + commit - scaled to one step."""
    import oracle
    p = step["params"]
    # this host's CPU share: OMP_NUM_THREADS where set, else every core we may run on
    threads = min(int(os.environ.get("OMP_NUM_THREADS") or 0) or 1 << 30, len(os.sched_getaffinity(0)))

    def attn(items):
        sl = lambda a: np.ascontiguousarray(a[items])
        oracle.attention(sl(step["q"]), sl(step["k_blk"]), sl(step["v_blk"]), sl(step["k_cache"]),
                         sl(step["v_cache"]), sl(step["prefix"]), p["mode"])

    def commit():
        oracle.confidence_commit(step["logits"], step["masked"], step["tokens"], p["S"], p["tau"])

    oracle.set_num_threads(threads)
    t0 = time.perf_counter()
    done = 0
    while True:
        attn(slice(None))
        commit()
        done += 1
        el = time.perf_counter() - t0
        if el >= budget_s / 2:
            break
    all_rate = done / el

    oracle.set_num_threads(1)
    sample_items = 2
    t0 = time.perf_counter()
    attn(slice(0, sample_items))
    ta = time.perf_counter() - t0
    t0 = time.perf_counter()
    commit()
    tc = time.perf_counter() - t0
    one_step_s = ta * p["n_items"] / sample_items + tc
    oracle.set_num_threads(threads)
    return dict(value=round(all_rate, 3), unit="steps/s", cores=threads, kind="oracle",
                sample="%d whole step(s) of the same workload (36-layer attention + confidence/commit) on %d "
                       "threads, %.1f s wall" % (done, threads, el),
                cpu_model=cpu_model(),
                single_thread=dict(value=round(1.0 / one_step_s, 4), unit="steps/s", cores=1,
                                   sample="attention of %d of the 36 layers (%.2f s, scaled x%d) + the whole "
                                          "confidence/commit (%.2f s), one thread" % (
                                              sample_items, ta, p["n_items"] // sample_items, tc)))


# ---------------------------------------------------------------------------
# rocprofv3 counter summaries -> committed traffic file
# ---------------------------------------------------------------------------

def _pmc_values(db_path, counter):
    """(kernel name, value) per dispatch of ``counter`` from a rocprofv3 database."""
    import sqlite3
    db = sqlite3.connect(db_path)
    rows = db.execute("select kernel_name, value, dispatch_id from counters_collection "
                      "where counter_name = ? order by dispatch_id", (counter,)).fetchall()
    db.close()
    return [(k, float(v)) for k, v, _ in rows]


def write_traffic(pmc_dir, copy_bytes=256 << 20):
    """HBM bytes per launch from four rocprofv3 --pmc runs in ``pmc_dir``:
    copyfetch/copywrite (FETCH_SIZE / WRITE_SIZE over --copy-calibration) give the
    counter-to-bytes scale; fetch/write (the same counters over a short bench run)
    give the attention and confidence kernels' readings, averaged over dispatches."""
    def scale(db, counter):
        vals = [v for k, v in _pmc_values(os.path.join(pmc_dir, db), counter) if "copyBuffer" in k]
        return copy_bytes / (sum(vals) / len(vals) * 1024.0)
    f_scale = scale("copyfetch_results.db", "FETCH_SIZE")
    w_scale = scale("copywrite_results.db", "WRITE_SIZE")
    per_kernel = {}
    for db, counter, sc in (("fetch_results.db", "FETCH_SIZE", f_scale), ("write_results.db", "WRITE_SIZE", w_scale)):
        acc = {}
        for k, v in _pmc_values(os.path.join(pmc_dir, db), counter):
            if "attn_" not in k and "row_kernel" not in k:
                continue
            name = k.replace("void bd::(anonymous namespace)::", "").split("(")[0]
            acc.setdefault(name, []).append(v * 1024.0 * sc)
        for name, vals in acc.items():
            per_kernel.setdefault(name, {})[counter.lower() + "_bytes"] = sum(vals) / len(vals)

    def launch_bytes(names):
        return sum(v.get("fetch_size_bytes", 0.0) + v.get("write_size_bytes", 0.0)
                   for k, v in per_kernel.items() if k in names)
    out = {
        "attn_bytes_per_launch": round(launch_bytes(HEADLINE_KERNELS)),
        "fp8kv_bytes_per_launch": round(launch_bytes(FP8KV_KERNELS)),
        "commit_bytes_per_launch": round(launch_bytes((ROW_KERNEL,))),
        "per_kernel": {k: {kk: round(vv) for kk, vv in v.items()} for k, v in per_kernel.items()},
        "fetch_scale": f_scale, "write_scale": w_scale,
        "calibration": "FETCH_SIZE/WRITE_SIZE over plain %d-byte device copies (bench.py --copy-calibration)" % copy_bytes,
        "attn_source_sha256": source_hash(ATTN_SOURCES),
        "row_source_sha256": source_hash(ROW_SOURCES),
    }
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def copy_calibration(n_bytes=256 << 20, reps=5):
    """Plain device-to-device copies of a known size: rocprofv3's FETCH_SIZE and
    WRITE_SIZE for this copy kernel give the scale between counter readings and
    bytes moved (each copy reads and writes n_bytes)."""
    import torch
    src = torch.ones(n_bytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n_bytes, "reps": reps}), flush=True)
    del src, dst


# ---------------------------------------------------------------------------
# Legs beside the headline
# ---------------------------------------------------------------------------

def attn_call(ds, desc=None):
    from vlm_decoding_amd import bd
    d = ds.adesc if desc is None else desc
    return (bd.lib.bd_attn_step, (ctypes.byref(d), ds.q.data_ptr(), ds.k_blk.data_ptr(), ds.v_blk.data_ptr(),
                                  ds.k_cache.data_ptr(), ds.v_cache.data_ptr(), ds.prefix.data_ptr(),
                                  ds.out.data_ptr(), ds.attn_ws.data_ptr(), ds.attn_ws.numel(),
                                  ds.stream_handle))


def commit_call(ds, masked_ptr=None, tokens_ptr=None):
    from vlm_decoding_amd import bd
    return (bd.lib.bd_confidence_commit,
            (ctypes.byref(ds.cdesc), ds.logits.data_ptr(), masked_ptr or ds.masked.data_ptr(),
             tokens_ptr or ds.tokens.data_ptr(), ds.conf.data_ptr(), ds.argmax.data_ptr(), ds.committed.data_ptr(),
             ds.n_committed.data_ptr(), ds.commit_ws.data_ptr(), ds.commit_ws.numel(), ds.stream_handle))


def leg_denoise_config(torch, stream, flush, cfg, iters, balanced=False):
    """One denoise step (attention + confidence/commit) of a configuration, timed
    cold: each iteration follows an untimed 1 GiB flush and starts from the
    initial block state.  ``balanced`` marks the batch as ragged (the attention
    plan then balances key splits across items from their prefix lengths)."""
    import synth
    from vlm_decoding_amd.step import DeviceStep
    st = synth.config_step(cfg)
    p = st["params"]
    ds = DeviceStep(st, balanced=balanced)
    ds.stream_handle = stream.cuda_stream
    ms = timed_calls(torch, stream, lambda i: [attn_call(ds), commit_call(ds)], iters, flush=flush,
                     before=lambda i: ds.reset_block_state())
    # A second pass with an event between the two calls, for each call's own time
    # (kept out of step_us, which the extra event would lengthen).
    a_ms, c_ms = timed_calls(torch, stream, lambda i: [attn_call(ds), commit_call(ds)], iters, flush=flush,
                             before=lambda i: ds.reset_block_state(), per_call=True)
    a_b = attn_bytes(p, st["prefix"])
    l_b, s_b = commit_bytes(p, int(st["masked"].sum()))
    total = a_b + l_b + s_b
    dist = dist_us(ms)
    med_s = dist["median"] * 1e-6
    a_d, c_d = dist_us(a_ms), dist_us(c_ms)
    per = lambda b, d: dict(us=d, gbps_at_median=round(b / (d["median"] * 1e-6) / 1e9, 1),
                            frac_at_median=round(b / (d["median"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4))
    out = dict(workload=p["name"] + (", ragged-batch plan (BD_PLAN_BALANCED)" if balanced else ""), step_us=dist,
               steps_per_s=round(1.0 / med_s, 1), algorithmic_bytes=total,
               attn_bytes=a_b, logits_bytes=l_b, achieved_gbps=round(total / med_s / 1e9, 1),
               frac=round(total / med_s / 1e9 / HBM_PEAK_GBS, 4),
               attention_call=per(a_b, a_d), commit_call=per(l_b + s_b, c_d),
               timing="cold: 1 GiB flush read before each step; the per-call times come from a second "
                      "pass with an event between the calls")
    del ds
    return out


def leg_verify_chain(torch, stream, flush, iters):
    """The 3B self-speculative verify chain of config 4, timed cold: causal block
    attention over the prefix of 2048, speculative verify of the 16 drafts over
    16 x 151936 logits, then the KV append of the accepted prefix (its length
    read on the device).  The append advances the prefix; it is restored
    outside the events."""
    import synth
    from vlm_decoding_amd import bd
    from vlm_decoding_amd.step import DeviceStep
    st = synth.config_step(4)
    p = st["params"]
    ds = DeviceStep(st)
    sh = stream.cuda_stream
    ds.stream_handle = sh
    prefix0 = ds.prefix.clone()
    verify = (bd.lib.bd_spec_verify, (p["n_req"], p["D"], p["V"], ds.logits.data_ptr(), ds.draft.data_ptr(),
                                      ds.accepted.data_ptr(), ds.argmax.data_ptr(), ds.verify_ws.data_ptr(),
                                      ds.verify_ws.numel(), sh))
    append = (bd.lib.bd_kv_append, (ctypes.byref(ds.adesc), ds.k_cache.data_ptr(), ds.v_cache.data_ptr(),
                                    ds.prefix.data_ptr(), ds.k_blk.data_ptr(), ds.v_blk.data_ptr(),
                                    ds.accepted.data_ptr(), ds.dev_err.data_ptr(), sh))
    ms = timed_calls(torch, stream, lambda i: [attn_call(ds), verify, append], iters, flush=flush,
                     before=lambda i: ds.prefix.copy_(prefix0))
    per_ms = timed_calls(torch, stream, lambda i: [attn_call(ds), verify, append], iters, flush=flush,
                         before=lambda i: ds.prefix.copy_(prefix0), per_call=True)
    L = int(ds.accepted.cpu()[0])
    assert L == int(st["planted_L"][0]) and int(ds.dev_err.cpu()[0]) == 0
    a_b = attn_bytes(p, st["prefix"])
    logits_read = p["n_req"] * p["D"] * p["V"] * 4
    logits_alg = min(L + 1, p["D"]) * p["V"] * 4
    app_b = L * p["Hkv"] * p["d"] * 2 * 2 * 2
    dist = dist_us(ms)
    med_s = dist["median"] * 1e-6
    total = a_b + logits_read + app_b
    out = dict(workload=p["name"], accepted_len=L, chain_us=dist, chains_per_s=round(1.0 / med_s, 1),
               attn_bytes=a_b, logits_bytes_read=logits_read, logits_bytes_algorithmic=logits_alg, append_bytes=app_b,
               algorithmic_bytes=total, achieved_gbps=round(total / med_s / 1e9, 1),
               frac=round(total / med_s / 1e9 / HBM_PEAK_GBS, 4),
               attention_us=dist_us(per_ms[0]), verify_us=dist_us(per_ms[1]), append_us=dist_us(per_ms[2]),
               timing="cold: 1 GiB flush read before each chain; all 16 logits rows read (verify needs every row "
                      "until the first mismatch is known on the device); the per-call times come from a second "
                      "pass with an event after each call")
    del ds
    return out


def bench_lmhead(torch, stream, iters=50, warmup=5):
    """The LM head (16 slots x 2048 hidden x 151936 vocabulary, bf16 weight of
    622 MB) fused with the confidence + commit of the 8 masked slots.  Each call
    starts from the same block state, restored outside the events."""
    import synth
    from vlm_decoding_amd import bd
    st = synth.lmhead_step(1)
    p = st["params"]
    c = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    hidden, weight = c(st["hidden"].view(np.int16)), c(st["weight"].view(np.int16))
    masked0, tokens0 = c(st["masked"]), c(st["tokens"])
    masked, tokens = masked0.clone(), tokens0.clone()
    nr, D = p["n_req"], p["D"]
    conf = torch.empty((nr, D), dtype=torch.float32, device="cuda")
    amax = torch.empty((nr, D), dtype=torch.int32, device="cuda")
    com = torch.empty((nr, D), dtype=torch.uint8, device="cuda")
    ncom = torch.empty((nr,), dtype=torch.int32, device="cuda")
    desc = bd.lmhead_desc(nr, D, p["V"], p["H"], p["S"], p["tau"])
    ws = torch.zeros(bd.bd_lmhead_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    args = (ctypes.byref(desc), hidden.data_ptr(), weight.data_ptr(), masked.data_ptr(), tokens.data_ptr(),
            conf.data_ptr(), amax.data_ptr(), com.data_ptr(), ncom.data_ptr(), ws.data_ptr(), ws.numel(),
            stream.cuda_stream)

    def restore(i):
        masked.copy_(masked0)
        tokens.copy_(tokens0)
    timed_calls(torch, stream, lambda i: [(bd.lib.bd_lmhead_confidence_commit, args)], warmup, before=restore)
    ms = timed_calls(torch, stream, lambda i: [(bd.lib.bd_lmhead_confidence_commit, args)], iters, before=restore)
    dist = dist_us(ms)
    nbytes = p["V"] * p["H"] * 2 + nr * D * p["H"] * 2
    return dict(workload="3B LM head: 16 slots x H 2048 x V 151936 bf16 (8 masked, S=16, tau=0.9)",
                us_per_call=dist, algorithmic_bytes=nbytes,
                achieved_gbps=round(nbytes / (dist["median"] * 1e-6) / 1e9, 1),
                frac=round(nbytes / (dist["median"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4))


def back_to_back(torch, stream, args_list, fn, calls, warmup):
    """Average time of ``calls`` calls issued back to back between two events,
    rotating over the argument tuples (the input sets)."""
    status = 0
    for i in range(warmup):
        status |= fn(*args_list[i % len(args_list)])
    ev = HipEvents(2)
    torch.cuda.synchronize()
    ev.record(0, stream.cuda_stream)
    for i in range(calls):
        status |= fn(*args_list[i % len(args_list)])
    ev.record(1, stream.cuda_stream)
    torch.cuda.synchronize()
    us = ev.ms(0, 1) * 1e3 / calls
    ev.destroy()
    if status:
        raise RuntimeError("a library call failed (status %d)" % status)
    return us


def bench_fp8kv_attention(torch, stream, calls=200, warmup=20):
    """The E4M3 KV-cache variant of the headline attention call: the same 36-layer
    3B-shape step (prefix 4096, D = 16) with keys and values stored as one byte
    each plus one fp32 scale per (layer, KV head).  Four input sets rotated; the
    calls run back to back between two events (tile kernel + merge per call)."""
    import synth
    from vlm_decoding_amd import bd
    from vlm_decoding_amd.step import DeviceStep
    p = synth.params_for(CFG, dtype=synth.FP8KV)
    sets = [DeviceStep(synth.make_step(p, synth.seed_of(CFG) + 1000 * k)) for k in range(N_SETS)]
    sh = stream.cuda_stream
    args = [(ctypes.byref(ds.adesc), ds.q.data_ptr(), ds.k_blk.data_ptr(), ds.v_blk.data_ptr(), ds.k_cache.data_ptr(),
             ds.v_cache.data_ptr(), ds.k_scale.data_ptr(), ds.v_scale.data_ptr(), ds.prefix.data_ptr(),
             ds.out.data_ptr(), ds.attn_ws.data_ptr(), ds.attn_ws.numel(), sh) for ds in sets]
    us = back_to_back(torch, stream, args, bd.lib.bd_attn_step_fp8kv, calls, warmup)
    prefix = sets[0].prefix.cpu().numpy()
    nbytes = attn_bytes(p, prefix, kv_elem=1) + p["n_items"] * p["Hkv"] * 2 * 4
    del sets
    return dict(workload="36 layers x block attention, 16q/2kv heads, d128, prefix 4096, D=16, "
                         "bf16 queries, E4M3 K/V cache with per-(layer, KV head) scales",
                us_per_call=round(us, 2), algorithmic_bytes=nbytes,
                achieved_gbps=round(nbytes / (us * 1e-6) / 1e9, 1),
                frac=round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), calls=calls,
                traffic=committed_traffic().get("fp8kv"))


def bench_quad_attention(torch, stream, calls=50, warmup=5):
    """The quadratic self-speculative step: 36 layers of the 3B shape (prefix 4096)
    with a draft block of B = 16, i.e. 152 block slots per layer (16 drafts + the
    mask tokens of 16 acceptance hypotheses), in one bd_attn_step call (mode
    BD_BLOCK_QUAD), beside the linear variant's two block passes (bidirectional
    draft + causal verify of the headline shape).  MFMA-bound: bf16 TFLOP/s over
    the algorithmic flops (4 d per visible (row, key) pair: the two products)."""
    import synth
    from vlm_decoding_amd import bd
    from vlm_decoding_amd.step import DeviceStep
    sh = stream.cuda_stream

    def args_of(ds, desc):
        return (ctypes.byref(desc), ds.q.data_ptr(), ds.k_blk.data_ptr(), ds.v_blk.data_ptr(), ds.k_cache.data_ptr(),
                ds.v_cache.data_ptr(), ds.prefix.data_ptr(), ds.out.data_ptr(), ds.attn_ws.data_ptr(),
                ds.attn_ws.numel(), sh)

    qsets = [DeviceStep(synth.make_quad_step(dict(synth.QUAD_CONFIGS[1]), synth.quad_seed_of(1) + 1000 * k))
             for k in range(N_SETS)]
    quad_us = back_to_back(torch, stream, [args_of(ds, ds.adesc) for ds in qsets], bd.lib.bd_attn_step, calls, warmup)
    p = qsets[0].p
    B, S, n, Hq, d = p["B"], p["D"], p["n_items"], p["Hq"], p["d"]
    P = int(qsets[0].prefix.cpu().numpy()[0])
    del qsets
    vis = S * P + sum(t + 1 for t in range(B)) + sum((B - g) * B for g in range(B))
    flops = 4.0 * d * vis * n * Hq
    lsets = [DeviceStep(synth.make_step(synth.params_for(CFG), synth.seed_of(CFG) + 1000 * k)) for k in range(N_SETS)]
    pair_args = []
    for ds in lsets:
        verify = bd.attn_desc(ds.adesc.n_items, ds.adesc.D, ds.adesc.Hq, ds.adesc.Hkv, ds.adesc.d, ds.adesc.cap,
                              ds.adesc.dtype, bd.BD_BLOCK_CAUSAL, ds.adesc.max_prefix)
        ds._verify_desc = verify
        pair_args += [args_of(ds, ds.adesc), args_of(ds, verify)]
    linear_us = 2 * back_to_back(torch, stream, pair_args, bd.lib.bd_attn_step, 2 * calls, 2 * warmup)
    del lsets
    tflops = flops / (quad_us * 1e-6) / 1e12
    return dict(workload="36 layers x quadratic speculative block attention, 16q/2kv heads, d128, bf16, prefix 4096, "
                         "B=16 (152 slots: 16 drafts + 136 mask tokens)",
                us_per_call=round(quad_us, 2), algorithmic_tflop=round(flops / 1e12, 4),
                achieved_tflops=round(tflops, 1), peak_tflops=MFMA_BF16_PEAK_TFLOPS,
                frac=round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                linear_draft_plus_verify_us=round(linear_us, 2), calls=calls)


def bench_two_stream(torch, stream, calls=30, warmup=3):
    """Two-stream training attention: the 3B training shape (8 sequences; clean
    stream 2048 = 1024 vision + two turns; noisy stream 832; D = 32; 16q/2kv,
    d = 128, bf16) in one bd_two_stream_attn call.  MFMA-bound: bf16 TFLOP/s over
    the algorithmic flops, 4 d per visible (row, key) pair."""
    import synth
    from vlm_decoding_amd import bd
    st = synth.two_stream_step(1)
    p = st["params"]
    n, L, Hq, d = st["q"].shape
    c = lambda a: torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if a.dtype == np.uint16 else a)).cuda()
    sets = []
    for k in range(N_SETS):
        s_k = st if k == 0 else synth.make_two_stream(p, synth.two_stream_seed_of(1) + 1000 * k)
        sets.append([c(s_k[x]) for x in ("q", "k", "v", "spans", "n_spans")])
    out = torch.empty_like(sets[0][0])
    desc = bd.two_stream_desc(n, st["Lc"], st["Ln"], st["cap"], p["D"], Hq, p["Hkv"], d, st["spans"].shape[1])
    ws = torch.zeros(max(bd.bd_two_stream_workspace_bytes(desc), 16), dtype=torch.uint8, device="cuda")
    args = [(ctypes.byref(desc), q.data_ptr(), k.data_ptr(), v.data_ptr(), sp.data_ptr(), ns.data_ptr(),
             out.data_ptr(), ws.data_ptr(), ws.numel(), stream.cuda_stream) for q, k, v, sp, ns in sets]
    us = back_to_back(torch, stream, args, bd.lib.bd_two_stream_attn, calls, warmup)
    Lc, D = st["Lc"], p["D"]
    vis = 0
    for it in range(n):
        pairs = Lc * (Lc + 1) // 2
        for c0, m in st["spans"][it, :st["n_spans"][it]]:
            for k0 in range(0, int(m), D):
                bl = min(D, int(m) - k0)
                pairs += bl * (int(c0) + k0 + bl)
        vis += pairs
    flops = 4.0 * d * vis * Hq
    tflops = flops / (us * 1e-6) / 1e12
    del sets, out, ws
    return dict(workload="two-stream training attention, 8 sequences x (clean 2048 = 1024 vision + 2 turns, "
                         "noisy 832), D=32, 16q/2kv, d128, bf16",
                us_per_call=round(us, 2), algorithmic_tflop=round(flops / 1e12, 4), achieved_tflops=round(tflops, 1),
                peak_tflops=MFMA_BF16_PEAK_TFLOPS, frac=round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), calls=calls)


def bench_layer_serial(torch, stream, sets, steps=100, warmup=5):
    """The headline step as a model runs it: the 36 layers' attention as 36
    dependent bd_attn_step launches of one layer each, then the confidence +
    commit, captured once per input set in a HIP graph (with two small copies
    that restore the block state) and replayed; each replay between events."""
    graphs = [ds.capture_layer_serial() for ds in sets]
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    ev = HipEvents(2 * steps)
    sh = stream.cuda_stream
    torch.cuda.synchronize()
    for i in range(steps):
        ev.record(2 * i, sh)
        graphs[i % len(graphs)].replay()
        ev.record(2 * i + 1, sh)
    torch.cuda.synchronize()
    dist = dist_us([ev.ms(2 * i, 2 * i + 1) for i in range(steps)])
    ev.destroy()
    del graphs
    gc.collect()
    return dict(workload="headline step, layer-serial: 36 x bd_attn_step(n_items=1) + bd_confidence_commit "
                         "in one HIP graph per input set",
                us_per_step=dist, steps_per_s=round(1e6 / dist["median"], 1),
                us_per_layer_call=round((dist["median"]) / 36.0, 2))


def copy_bandwidth(torch, n_bytes=1 << 30, reps=5):
    """Measured device-to-device copy rate (torch copy of 1 GiB, read + write),
    the practical HBM ceiling the roofline fractions can be read against."""
    src = torch.ones(n_bytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    ev = HipEvents(2)
    torch.cuda.synchronize()
    ev.record(0, torch.cuda.current_stream().cuda_stream)
    for _ in range(reps):
        dst.copy_(src)
    ev.record(1, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    gbps = 2 * n_bytes * reps / (ev.ms(0, 1) * 1e-3) / 1e9
    ev.destroy()
    del src, dst
    return round(gbps, 1)


# ---------------------------------------------------------------------------
# The headline
# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--event-samples", type=int, default=200,
                    help="steps of the sampled pass after the timed region, each call between events (at least 20)")
    ap.add_argument("--cold-steps", type=int, default=100,
                    help="headline steps timed one by one after a 1 GiB flush (0 to skip)")
    ap.add_argument("--config-iters", type=int, default=40,
                    help="cold iterations of the other configurations' legs (0 to skip)")
    ap.add_argument("--lmhead-calls", type=int, default=50,
                    help="timed calls of the fused LM head + confidence + commit (0 to skip)")
    ap.add_argument("--fp8kv-calls", type=int, default=200,
                    help="timed calls of the E4M3 KV-cache attention variant (0 to skip)")
    ap.add_argument("--quad-calls", type=int, default=50,
                    help="timed calls of the quadratic self-speculative attention step (0 to skip)")
    ap.add_argument("--two-stream-calls", type=int, default=30,
                    help="timed calls of the two-stream training attention (0 to skip)")
    ap.add_argument("--layer-serial-steps", type=int, default=100,
                    help="timed replays of the layer-serial graph of the headline step (0 to skip)")
    ap.add_argument("--cpu-budget", type=float, default=20.0,
                    help="seconds of oracle work for cpu_baseline (0 to skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain 256 MiB device copies (to scale HBM byte counters)")
    ap.add_argument("--traffic-from", metavar="DIR",
                    help="summarise rocprofv3 --pmc databases in DIR into the committed traffic file")
    args = ap.parse_args()
    if args.traffic_from:
        write_traffic(args.traffic_from)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import torch
    import synth
    from vlm_decoding_amd import bd
    from vlm_decoding_amd.step import DeviceStep

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    p = synth.params_for(CFG)
    sets = []
    host0 = None
    for k in range(N_SETS):
        s = synth.make_step(p, synth.seed_of(CFG) + 1000 * k)
        if k == 0:
            host0 = s
        sets.append(DeviceStep(s))
        print("input set %d uploaded" % k, file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    for ds in sets:
        ds.stream_handle = sh
    # The commit mutates the block state (masked flags, tokens), so every step
    # gets its own copy of its set's initial state, prepared before timing: one
    # 128-byte row per step (masked at bytes 0..15, tokens at 64..127).
    n_samples = max(20, args.event_samples)
    total = args.warmup + args.steps + n_samples
    rows = np.zeros((N_SETS, 128), dtype=np.uint8)
    for k, ds in enumerate(sets):
        rows[k, :16] = ds.masked0.cpu().numpy().reshape(-1)
        rows[k, 64:128] = ds.tokens0.cpu().numpy().reshape(-1).view(np.uint8)
    state = torch.from_numpy(rows[np.arange(total) % N_SETS]).to("cuda")
    torch.cuda.synchronize()

    a_bytes = attn_bytes(p, host0["prefix"])
    l_bytes, s_bytes = commit_bytes(p, int(host0["masked"].sum()))
    step_bytes = a_bytes + l_bytes + s_bytes

    # The timed loop calls the C ABI directly with argument tuples prepared here
    # (raw device pointers, the stream handle), so that enqueueing a step costs
    # the host far less than the step costs the GPU.
    attn_args = [attn_call(ds)[1] for ds in sets]
    base = state.data_ptr()
    commit_args = [commit_call(sets[i % N_SETS], base + 128 * i, base + 128 * i + 64)[1] for i in range(total)]
    attn_fn, commit_fn = bd.lib.bd_attn_step, bd.lib.bd_confidence_commit

    status = 0
    for i in range(args.warmup):
        status |= attn_fn(*attn_args[i % N_SETS])
        status |= commit_fn(*commit_args[i])
    torch.cuda.synchronize()
    if status:
        raise RuntimeError("a library call failed during warm-up (status %d)" % status)
    # The timed region: exactly K steps, with one event pair around all of them
    # (per-call events inside it would add their own records to the GPU's work).
    ev = HipEvents(2)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev.record(0, sh)
    for i in range(args.steps):
        j = args.warmup + i
        status |= attn_fn(*attn_args[j % N_SETS])
        status |= commit_fn(*commit_args[j])
    ev.record(1, sh)
    t_enq = time.perf_counter() - t0
    # The clock stops when the last event is seen complete by polling: a blocking
    # synchronize wakes the host up to several ms late now and then, which would
    # be timed as GPU work.
    ev.wait(1)
    elapsed = time.perf_counter() - t0
    torch.cuda.synchronize()
    if status:
        raise RuntimeError("a library call failed in the timed loop (status %d)" % status)
    gpu_ms_per_step = ev.ms(0, 1) / args.steps
    ev.destroy()
    # The sampled pass, after the timed region and not part of `value`: the same
    # step, each call between events, for the per-call distributions.
    ev = HipEvents(3 * n_samples)
    for n in range(n_samples):
        j = args.warmup + args.steps + n
        ev.record(3 * n, sh)
        status |= attn_fn(*attn_args[j % N_SETS])
        ev.record(3 * n + 1, sh)
        status |= commit_fn(*commit_args[j])
        ev.record(3 * n + 2, sh)
    torch.cuda.synchronize()
    if status:
        raise RuntimeError("a library call failed in the sampled pass (status %d)" % status)
    attn_ms = [ev.ms(3 * n, 3 * n + 1) for n in range(n_samples)]
    conf_ms = [ev.ms(3 * n + 1, 3 * n + 2) for n in range(n_samples)]
    step_ms = [ev.ms(3 * n, 3 * n + 2) for n in range(n_samples)]
    ev.destroy()
    ms_per_step = elapsed * 1e3 / args.steps
    attn_d, conf_d, step_d = dist_us(attn_ms), dist_us(conf_ms), dist_us(step_ms)
    attn_avg_s = attn_d["mean"] * 1e-6
    achieved = a_bytes / attn_avg_s / 1e9
    traffic = committed_traffic()

    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic.get("attn"),
                    kernel="bd_attn_step (%s + %s)" % HEADLINE_KERNELS,
                    kernel_avg_us=attn_d["mean"], kernel_us=attn_d,
                    algorithmic_bytes_per_launch=a_bytes,
                    achieved_at_median_gbps=round(a_bytes / (attn_d["median"] * 1e-6) / 1e9, 1))

    flush = torch.zeros(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    cold = None
    if args.cold_steps > 0:
        ds0 = sets[0]
        cold_ms = timed_calls(torch, stream, lambda i: [attn_call(ds0), commit_call(ds0)], args.cold_steps,
                              flush=flush, before=lambda i: ds0.reset_block_state())
        cd = dist_us(cold_ms)
        cold = dict(step_us=cd, steps_per_s=round(1e6 / cd["median"], 1),
                    step_gbps=round(step_bytes / (cd["median"] * 1e-6) / 1e9, 1),
                    step_frac=round(step_bytes / (cd["median"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                    timing="each step alone after an untimed 1 GiB flush read, between HIP events")
    configs = None
    if args.config_iters > 0:
        configs = {"cfg2_3b_single_layer": leg_denoise_config(torch, stream, flush, 2, args.config_iters),
                   "cfg4_3b_verify_chain": leg_verify_chain(torch, stream, flush, args.config_iters),
                   "cfg5_7b_batched": leg_denoise_config(torch, stream, flush, 5, args.config_iters, balanced=True),
                   "cfg5_7b_batched_plain_plan": leg_denoise_config(torch, stream, flush, 5, args.config_iters)}
    del flush

    layer_serial = (bench_layer_serial(torch, stream, sets, steps=args.layer_serial_steps)
                    if args.layer_serial_steps > 0 else None)
    del sets, state, attn_args, commit_args
    gc.collect()
    torch.cuda.empty_cache()
    copy_gbps = copy_bandwidth(torch)
    roofline["copy_gbps_measured"] = copy_gbps
    roofline["frac_of_copy"] = round(achieved / copy_gbps, 4)
    lmhead = bench_lmhead(torch, stream, iters=args.lmhead_calls) if args.lmhead_calls > 0 else None
    fp8kv = bench_fp8kv_attention(torch, stream, calls=args.fp8kv_calls) if args.fp8kv_calls > 0 else None
    quad = bench_quad_attention(torch, stream, calls=args.quad_calls) if args.quad_calls > 0 else None
    two_stream = bench_two_stream(torch, stream, calls=args.two_stream_calls) if args.two_stream_calls > 0 else None

    cpu = cpu_baseline(host0, args.cpu_budget) if args.cpu_budget > 0 else None

    steps_per_s = args.steps / elapsed
    out = {
        "metric": METRIC,
        "value": round(steps_per_s, 1),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "3B-shape long-reasoning denoise step: 36 layers x block attention "
                        "(16q/2kv heads, d128, bf16, prefix 4096, block D=16, 8 of 16 masked) + "
                        "confidence/commit over 8 x 151936 fp32 logits (S=16, tau=0.9)",
            "layers": p["n_items"], "prefix": 4096, "block": p["D"], "heads_q": p["Hq"], "heads_kv": p["Hkv"],
            "head_dim": p["d"], "vocab": p["V"], "masked": int(host0["masked"].sum()), "S": p["S"],
            "tau": p["tau"], "input_sets_rotated": N_SETS,
        },
        "step_hbm_gbps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "step_hbm_frac": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "algorithmic_bytes_per_step": step_bytes,
        "step_us": step_d,
        "confidence_commit_us": conf_d,
        "confidence_commit_algorithmic_bytes": l_bytes + s_bytes,
        "confidence_commit_gbps_at_median": round((l_bytes + s_bytes) / (conf_d["median"] * 1e-6) / 1e9, 1),
        "confidence_commit_traffic": traffic.get("commit"),
        "host_enqueue_us_per_step": round(t_enq * 1e6 / args.steps, 2),
        "gpu_event_us_per_step": round(gpu_ms_per_step * 1e3, 2),
        "event_samples": n_samples,
        "steps_per_s_at_median": round(1e6 / step_d["median"], 1),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "cold_step": cold,
        "configs": configs,
        "layer_serial_graph": layer_serial,
        "lm_head_confidence_commit": lmhead,
        "fp8kv_attention": fp8kv,
        "quad_spec_attention": quad,
        "two_stream_attention": two_stream,
    }
    print(json.dumps(out), flush=True)
    # Leave nothing for interpreter teardown to release: every device object is
    # dropped and the device drained here, while the HIP runtime is whole.
    del out
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
