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

Prints one JSON line (see the keys below).  ``roofline`` describes the
attention call (the dominant one): algorithmic bytes per launch divided by
its average duration from HIP events recorded on the launch stream around
the calls of every 10th timed step (--event-stride; an event record costs the
GPU a few microseconds, so instrumenting every step would slow the steps it
measures).  ``value`` is steps over the wall time of all timed steps.
``cpu_baseline`` times the fp64 CPU oracle on the host.  Two further legs
measure the next rows of the path beside the headline: the LM head fused with
the confidence + commit (``lm_head_confidence_commit``) and the same attention
call over an E4M3 KV cache (``fp8kv_attention``), and the quadratic
self-speculative step (``quad_spec_attention``), and the two-stream training
attention (``two_stream_attention``).
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

CFG = 3
N_SETS = 4
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA, MI355X
METRIC = "denoise steps/sec + achieved HBM GB/s (%peak), 3B-shape block-16, 1 GPU"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_cfg3_traffic.json")
HEADLINE_KERNELS = ("attn_mfma_kernel<128, 4, false, false>", "attn_merge_kernel<128, 4, 32, false, 4, 16, 1>")
FP8KV_KERNELS = ("attn_mfma_kernel<128, 4, true, false>", "attn_merge_kernel<128, 4, 64, false, 4, 16, 1>")
ATTN_SOURCES = ["vlm_decoding_amd/csrc/bd_attn.hip", "vlm_decoding_amd/csrc/bd_common.h",
                "vlm_decoding_amd/csrc/bd_internal.h"]


def algorithmic_bytes(p, prefix, n_masked):
    """Bytes a step must move at least once: every K/V element of the prefix and the
    block once per KV head, Q read, O written, and the masked rows' logits."""
    n, D, Hq, Hkv, d = p["n_items"], p["D"], p["Hq"], p["Hkv"], p["d"]
    kv = int(np.sum(prefix.astype(np.int64) + D)) * Hkv * d * 2 * 2
    qo = n * D * Hq * d * 2 * 2
    logits = n_masked * p["V"] * 4
    state = D * (1 + 4) * 2 + D * (4 + 4 + 1) + 4   # masked/tokens in+out, conf/argmax/committed, count
    return kv + qo, logits, state


def attn_source_hash():
    h = hashlib.sha256()
    for rel in ATTN_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_per_launch(key="bytes_per_launch"):
    """HBM bytes per attention launch from committed counter runs, if they still
    describe the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != attn_source_hash():
        return None
    return t.get(key)


def cpu_baseline(step, budget_s):
    """The fp64 oracle on the host cores: whole steps (36-layer attention, then
    confidence + commit) repeated until ``budget_s`` of wall time has passed."""
    import oracle
    p = step["params"]
    t0 = time.perf_counter()
    done = 0
    while True:
        oracle.attention(step["q"], step["k_blk"], step["v_blk"], step["k_cache"], step["v_cache"],
                         step["prefix"], p["mode"])
        oracle.confidence_commit(step["logits"], step["masked"], step["tokens"], p["S"], p["tau"])
        done += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return dict(value=done / el, unit="steps/s", cores=oracle.num_threads(), kind="oracle",
                sample="%d full step(s) of the same workload (36-layer attention + confidence/commit), "
                       "%.1f s wall" % (done, el))


def _pmc_values(db_path, counter):
    """(kernel name, value) per dispatch of ``counter`` from a rocprofv3 database."""
    import sqlite3
    db = sqlite3.connect(db_path)
    rows = db.execute("select kernel_name, value, dispatch_id from counters_collection "
                      "where counter_name = ? order by dispatch_id", (counter,)).fetchall()
    db.close()
    return [(k, float(v)) for k, v, _ in rows]


def write_traffic(pmc_dir, copy_bytes=256 << 20):
    """HBM bytes per bd_attn_step launch from four rocprofv3 --pmc runs in ``pmc_dir``:
    copyfetch/copywrite (FETCH_SIZE / WRITE_SIZE over --copy-calibration) give the
    counter-to-bytes scale; fetch/write (the same counters over a short bench run)
    give the attention kernels' readings, averaged over their dispatches."""
    def scale(db, counter):
        vals = [v for k, v in _pmc_values(os.path.join(pmc_dir, db), counter) if "copyBuffer" in k]
        return copy_bytes / (sum(vals) / len(vals) * 1024.0)
    f_scale = scale("copyfetch_results.db", "FETCH_SIZE")
    w_scale = scale("copywrite_results.db", "WRITE_SIZE")
    per_kernel = {}
    for db, counter, sc in (("fetch_results.db", "FETCH_SIZE", f_scale), ("write_results.db", "WRITE_SIZE", w_scale)):
        acc = {}
        for k, v in _pmc_values(os.path.join(pmc_dir, db), counter):
            if "attn_" not in k:
                continue
            name = k.replace("void bd::(anonymous namespace)::", "").split("(")[0]
            acc.setdefault(name, []).append(v * 1024.0 * sc)
        for name, vals in acc.items():
            per_kernel.setdefault(name, {})[counter.lower() + "_bytes"] = sum(vals) / len(vals)
    # The headline call is the bf16 block-mode instance pair; the E4M3 pair is
    # summed on its own.
    def launch_bytes(names):
        return sum(v.get("fetch_size_bytes", 0.0) + v.get("write_size_bytes", 0.0)
                   for k, v in per_kernel.items() if k in names)
    out = {
        "bytes_per_launch": round(launch_bytes(HEADLINE_KERNELS)),
        "fp8kv_bytes_per_launch": round(launch_bytes(FP8KV_KERNELS)),
        "per_kernel": {k: {kk: round(vv) for kk, vv in v.items()} for k, v in per_kernel.items()},
        "fetch_scale": f_scale, "write_scale": w_scale,
        "calibration": "FETCH_SIZE/WRITE_SIZE over plain %d-byte device copies (bench.py --copy-calibration)" % copy_bytes,
        "kernel_source_sha256": attn_source_hash(),
    }
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def bench_lmhead(torch, stream, calls=50, warmup=5):
    """The next step of the path, measured beside the headline: the 3B LM head
    (16 slots x 2048 hidden x 151936 vocabulary, bf16 weight of 622 MB) fused with
    the confidence + commit of the 8 masked slots.  Each call starts from the same
    block state (restored by a small device copy outside the timed events)."""
    import ctypes
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
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    status = 0
    for i in range(warmup + calls):
        masked.copy_(masked0)
        tokens.copy_(tokens0)
        if i >= warmup:
            evs[i - warmup][0].record(stream)
        status |= bd.lib.bd_lmhead_confidence_commit(*args)
        if i >= warmup:
            evs[i - warmup][1].record(stream)
    torch.cuda.synchronize()
    if status:
        raise RuntimeError("bd_lmhead_confidence_commit failed (status %d)" % status)
    us = float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3
    nbytes = p["V"] * p["H"] * 2 + nr * D * p["H"] * 2
    return dict(workload="3B LM head: 16 slots x H 2048 x V 151936 bf16 (8 masked, S=16, tau=0.9)",
                us_per_call=round(us, 2), algorithmic_bytes=nbytes,
                achieved_gbps=round(nbytes / (us * 1e-6) / 1e9, 1),
                frac=round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), calls=calls)


def bench_fp8kv_attention(torch, stream, calls=200, warmup=20):
    """The E4M3 KV-cache variant of the headline attention call, measured beside it:
    the same 36-layer 3B-shape step (prefix 4096, D = 16) with keys and values stored
    as one byte each plus one fp32 scale per (layer, KV head).  Four input sets are
    rotated as in the main loop; the timed calls run back to back between two
    events, so the figure is the average launch-to-launch time of one call (tile
    kernel + merge)."""
    import ctypes
    import synth
    from vlm_decoding_amd import bd
    from vlm_decoding_amd.step import DeviceStep
    p = synth.params_for(CFG, dtype=synth.FP8KV)
    sets = [DeviceStep(synth.make_step(p, synth.seed_of(CFG) + 1000 * k)) for k in range(N_SETS)]
    sh = stream.cuda_stream
    args = [(ctypes.byref(ds.adesc), ds.q.data_ptr(), ds.k_blk.data_ptr(), ds.v_blk.data_ptr(), ds.k_cache.data_ptr(),
             ds.v_cache.data_ptr(), ds.k_scale.data_ptr(), ds.v_scale.data_ptr(), ds.prefix.data_ptr(),
             ds.out.data_ptr(), ds.attn_ws.data_ptr(), ds.attn_ws.numel(), sh) for ds in sets]
    call = bd.lib.bd_attn_step_fp8kv
    status = 0
    for i in range(warmup):
        status |= call(*args[i % N_SETS])
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(calls):
        status |= call(*args[i % N_SETS])
    t1.record(stream)
    torch.cuda.synchronize()
    if status:
        raise RuntimeError("bd_attn_step_fp8kv failed (status %d)" % status)
    us = t0.elapsed_time(t1) * 1e3 / calls
    prefix = sets[0].prefix.cpu().numpy()
    n, D, Hq, Hkv, d = p["n_items"], p["D"], p["Hq"], p["Hkv"], p["d"]
    nbytes = int(np.sum(prefix.astype(np.int64) + D)) * Hkv * d * 2 + n * D * Hq * d * 2 * 2 + n * Hkv * 2 * 4
    return dict(workload="36 layers x block attention, 16q/2kv heads, d128, prefix 4096, D=16, "
                         "bf16 queries, E4M3 K/V cache with per-(layer, KV head) scales",
                us_per_call=round(us, 2), algorithmic_bytes=nbytes,
                achieved_gbps=round(nbytes / (us * 1e-6) / 1e9, 1),
                frac=round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), calls=calls,
                traffic=traffic_per_launch("fp8kv_bytes_per_launch"))


def bench_quad_attention(torch, stream, calls=50, warmup=5):
    """The quadratic self-speculative step beside the headline: 36 layers of the
    3B shape (prefix 4096) with a draft block of B = 16, i.e. 152 block slots per
    layer (16 drafts + the mask tokens of 16 acceptance hypotheses), in one
    bd_attn_step call (mode BD_BLOCK_QUAD).  The linear variant needs two block
    passes for the same block, a bidirectional draft and a causal verify, each of
    the headline call's shape; both are timed here the same way for comparison.
    Work is MFMA-bound: the figure of merit is bf16 TFLOP/s over the algorithmic
    flops (4 d per visible (row, key) pair: the two products)."""
    import ctypes
    import synth
    from vlm_decoding_amd import bd
    from vlm_decoding_amd.step import DeviceStep
    sh = stream.cuda_stream

    def timed(args_list, n_calls):
        status = 0
        for i in range(warmup):
            for a in args_list[i % len(args_list)]:
                status |= bd.lib.bd_attn_step(*a)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for i in range(n_calls):
            for a in args_list[i % len(args_list)]:
                status |= bd.lib.bd_attn_step(*a)
        t1.record(stream)
        torch.cuda.synchronize()
        if status:
            raise RuntimeError("bd_attn_step failed (status %d)" % status)
        return t0.elapsed_time(t1) * 1e3 / n_calls

    def args_of(ds, desc):
        return (ctypes.byref(desc), ds.q.data_ptr(), ds.k_blk.data_ptr(), ds.v_blk.data_ptr(), ds.k_cache.data_ptr(),
                ds.v_cache.data_ptr(), ds.prefix.data_ptr(), ds.out.data_ptr(), ds.attn_ws.data_ptr(),
                ds.attn_ws.numel(), sh)

    qsets = [DeviceStep(synth.make_quad_step(dict(synth.QUAD_CONFIGS[1]), synth.quad_seed_of(1) + 1000 * k))
             for k in range(N_SETS)]
    quad_us = timed([[args_of(ds, ds.adesc)] for ds in qsets], calls)
    p = qsets[0].p
    B, S, n, Hq, d = p["B"], p["D"], p["n_items"], p["Hq"], p["d"]
    P = int(qsets[0].prefix.cpu().numpy()[0])
    del qsets
    # Visible keys summed over the slots of one (item, head): every slot sees the
    # prefix; draft t sees t + 1 drafts; a mask token of group g sees g drafts
    # and the B - g mask tokens of its group.
    vis = S * P + sum(t + 1 for t in range(B)) + sum((B - g) * B for g in range(B))
    flops = 4.0 * d * vis * n * Hq
    lsets = [DeviceStep(synth.make_step(synth.params_for(CFG), synth.seed_of(CFG) + 1000 * k)) for k in range(N_SETS)]
    pairs = []
    for ds in lsets:
        verify = bd.attn_desc(ds.adesc.n_items, ds.adesc.D, ds.adesc.Hq, ds.adesc.Hkv, ds.adesc.d, ds.adesc.cap,
                              ds.adesc.dtype, bd.BD_BLOCK_CAUSAL, ds.adesc.max_prefix)
        ds._verify_desc = verify
        pairs.append([args_of(ds, ds.adesc), args_of(ds, verify)])
    linear_us = timed(pairs, calls)
    tflops = flops / (quad_us * 1e-6) / 1e12
    return dict(workload="36 layers x quadratic speculative block attention, 16q/2kv heads, d128, bf16, prefix 4096, "
                         "B=16 (152 slots: 16 drafts + 136 mask tokens)",
                us_per_call=round(quad_us, 2), algorithmic_tflop=round(flops / 1e12, 4),
                achieved_tflops=round(tflops, 1), peak_tflops=MFMA_BF16_PEAK_TFLOPS,
                frac=round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                linear_draft_plus_verify_us=round(linear_us, 2), calls=calls)


def bench_two_stream(torch, stream, calls=30, warmup=3):
    """Two-stream training attention beside the headline: the 3B training shape
    (8 sequences; clean stream 2048 = 1024 vision + two turns; noisy stream 832;
    D = 32; 16q/2kv, d = 128, bf16) in one bd_two_stream_attn call.  MFMA-bound:
    the figure of merit is bf16 TFLOP/s over the algorithmic flops, 4 d per
    visible (row, key) pair."""
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
    import ctypes
    args = [(ctypes.byref(desc), q.data_ptr(), k.data_ptr(), v.data_ptr(), sp.data_ptr(), ns.data_ptr(),
             out.data_ptr(), ws.data_ptr(), ws.numel(), stream.cuda_stream) for q, k, v, sp, ns in sets]
    status = 0
    for i in range(warmup):
        status |= bd.lib.bd_two_stream_attn(*args[i % N_SETS])
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(calls):
        status |= bd.lib.bd_two_stream_attn(*args[i % N_SETS])
    t1.record(stream)
    torch.cuda.synchronize()
    if status:
        raise RuntimeError("bd_two_stream_attn failed (status %d)" % status)
    us = t0.elapsed_time(t1) * 1e3 / calls
    # Visible (row, key) pairs per head: clean rows see 1..Lc keys; a noisy block
    # row sees the clean positions before its block plus its block.
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
    return dict(workload="two-stream training attention, 8 sequences x (clean 2048 = 1024 vision + 2 turns, "
                         "noisy 832), D=32, 16q/2kv, d128, bf16",
                us_per_call=round(us, 2), algorithmic_tflop=round(flops / 1e12, 4), achieved_tflops=round(tflops, 1),
                peak_tflops=MFMA_BF16_PEAK_TFLOPS, frac=round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), calls=calls)


def bench_layer_serial(torch, stream, sets, steps=100, warmup=5):
    """The headline step as a model runs it, beside the batched headline: the 36
    layers' attention as 36 dependent bd_attn_step launches of one layer each, then
    the confidence + commit, captured once per input set in a HIP graph (with two
    small copies that restore the block state) and replayed."""
    graphs = [ds.capture_layer_serial() for ds in sets]
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    t1.record(stream)
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / steps
    return dict(workload="headline step, layer-serial: 36 x bd_attn_step(n_items=1) + bd_confidence_commit "
                         "in one HIP graph per input set",
                us_per_step=round(us, 2), steps_per_s=round(1e6 / us, 1), steps=steps)


def copy_bandwidth(torch, n_bytes=1 << 30, reps=5):
    """Measured device-to-device copy rate (torch copy of 1 GiB, read + write),
    the practical HBM ceiling the roofline fractions can be read against."""
    src = torch.ones(n_bytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(reps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    gbps = 2 * n_bytes * reps / (t0.elapsed_time(t1) * 1e-3) / 1e9
    del src, dst
    return round(gbps, 1)


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--event-stride", type=int, default=10,
                    help="record the per-call HIP events on every N-th timed step (0: none)")
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
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for cpu_baseline (0 to skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain 256 MiB device copies (to scale HBM byte counters)")
    ap.add_argument("--traffic-from", metavar="DIR",
                    help="summarise rocprofv3 --pmc databases in DIR into the committed traffic file")
    args = ap.parse_args()
    if args.traffic_from:
        write_traffic(args.traffic_from)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
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
    # The commit mutates the block state (masked flags, tokens), so every step
    # gets its own copy of its set's initial state, prepared before timing: one
    # 128-byte row per step (masked at bytes 0..15, tokens at 64..127).
    total = args.warmup + args.steps
    rows = np.zeros((N_SETS, 128), dtype=np.uint8)
    for k, ds in enumerate(sets):
        rows[k, :16] = ds.masked0.cpu().numpy().reshape(-1)
        rows[k, 64:128] = ds.tokens0.cpu().numpy().reshape(-1).view(np.uint8)
    state = torch.from_numpy(rows[np.arange(total) % N_SETS]).to("cuda")
    torch.cuda.synchronize()

    attn_bytes, logit_bytes, state_bytes = algorithmic_bytes(p, host0["prefix"], int(host0["masked"].sum()))
    step_bytes = attn_bytes + logit_bytes + state_bytes
    stream = torch.cuda.current_stream()

    # The timed loop calls the C ABI directly with argument tuples prepared
    # here (raw device pointers, the stream handle), so that enqueueing a step
    # costs the host far less than the step costs the GPU and the GPU never
    # waits for the host.  Step i uses its own state row (masked at +0, tokens
    # at +64).
    import ctypes
    from vlm_decoding_amd import bd
    lib = bd.lib
    sh = stream.cuda_stream
    attn_args = [(ctypes.byref(ds.adesc), ds.q.data_ptr(), ds.k_blk.data_ptr(), ds.v_blk.data_ptr(),
                  ds.k_cache.data_ptr(), ds.v_cache.data_ptr(), ds.prefix.data_ptr(), ds.out.data_ptr(),
                  ds.attn_ws.data_ptr(), ds.attn_ws.numel(), sh) for ds in sets]
    base = state.data_ptr()
    commit_args = []
    for i in range(total):
        ds = sets[i % N_SETS]
        commit_args.append((ctypes.byref(ds.cdesc), ds.logits.data_ptr(), base + 128 * i, base + 128 * i + 64,
                            ds.conf.data_ptr(), ds.argmax.data_ptr(), ds.committed.data_ptr(),
                            ds.n_committed.data_ptr(), ds.commit_ws.data_ptr(), ds.commit_ws.numel(), sh))
    attn_call, commit_call = lib.bd_attn_step, lib.bd_confidence_commit

    status = 0
    for i in range(args.warmup):
        status |= attn_call(*attn_args[i % N_SETS])
        status |= commit_call(*commit_args[i])
    torch.cuda.synchronize()
    if status:
        raise RuntimeError("a library call failed during warm-up (status %d)" % status)
    stride = args.event_stride
    timed = [i for i in range(args.steps) if stride > 0 and i % stride == 0]
    evs = {i: tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for i in timed}
    t_begin, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_begin.record(stream)
    for i in range(args.steps):
        j = args.warmup + i
        ev = evs.get(i)
        if ev is None:
            status |= attn_call(*attn_args[j % N_SETS])
            status |= commit_call(*commit_args[j])
            continue
        ev[0].record(stream)
        status |= attn_call(*attn_args[j % N_SETS])
        ev[1].record(stream)
        status |= commit_call(*commit_args[j])
        ev[2].record(stream)
    t_end.record(stream)
    t_enq = time.perf_counter() - t0
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    if status:
        raise RuntimeError("a library call failed in the timed loop (status %d)" % status)
    ms_per_step = elapsed * 1e3 / args.steps
    gpu_ms_per_step = t_begin.elapsed_time(t_end) / args.steps
    if not evs:
        raise SystemExit("--event-stride 0 leaves no per-call timing; use a stride >= 1")
    attn_ms = np.array([a.elapsed_time(b) for a, b, _ in evs.values()])
    conf_ms = np.array([b.elapsed_time(c) for _, b, c in evs.values()])
    attn_avg_s = float(attn_ms.mean()) * 1e-3
    achieved = attn_bytes / attn_avg_s / 1e9

    tr = traffic_per_launch()
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=tr,
                    kernel="bd_attn_step (%s + %s)" % HEADLINE_KERNELS,
                    kernel_avg_us=round(attn_avg_s * 1e6, 2),
                    kernel_p10_p90_us=[round(float(np.percentile(attn_ms, 10)) * 1e3, 2),
                                       round(float(np.percentile(attn_ms, 90)) * 1e3, 2)],
                    algorithmic_bytes_per_launch=attn_bytes)

    layer_serial = (bench_layer_serial(torch, stream, sets, steps=args.layer_serial_steps)
                    if args.layer_serial_steps > 0 else None)
    copy_gbps = copy_bandwidth(torch)
    roofline["copy_gbps_measured"] = copy_gbps
    roofline["frac_of_copy"] = round(achieved / copy_gbps, 4)
    lmhead = bench_lmhead(torch, stream, calls=args.lmhead_calls) if args.lmhead_calls > 0 else None
    fp8kv = bench_fp8kv_attention(torch, stream, calls=args.fp8kv_calls) if args.fp8kv_calls > 0 else None
    quad = bench_quad_attention(torch, stream, calls=args.quad_calls) if args.quad_calls > 0 else None
    two_stream = bench_two_stream(torch, stream, calls=args.two_stream_calls) if args.two_stream_calls > 0 else None

    cpu = None
    if args.cpu_budget > 0:
        cpu = cpu_baseline(host0, args.cpu_budget)

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
        "confidence_commit_avg_us": round(float(conf_ms.mean()) * 1e3, 2),
        "host_enqueue_us_per_step": round(t_enq * 1e6 / args.steps, 2),
        "gpu_event_us_per_step": round(gpu_ms_per_step * 1e3, 2),
        "event_stride": stride,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "layer_serial_graph": layer_serial,
        "lm_head_confidence_commit": lmhead,
        "fp8kv_attention": fp8kv,
        "quad_spec_attention": quad,
        "two_stream_attention": two_stream,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
