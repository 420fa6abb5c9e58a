#!/usr/bin/env python3
"""Benchmark: effective KV-cache read GB/s (fraction of MI355X HBM peak) and
us per decode step of paged decode attention on one GPU.

Default workload: GQA decode at batch, B=64, Hq=32, Hkv=8, d=128, every context
1024 tokens, page 16, fp16 cache and queries ~ N(0, 1), block tables a random
permutation of a 4096-page pool, no split-KV; the cache pages are head-major
([pages, Hkv, P, d], one KV head's 16 rows of a page contiguous).  The same
cache with token-major pages ([pages, P, Hkv, d]) is measured as "gqa_b64"
among the other workloads.

A step is one call of the C-ABI entry point (planner + attention kernel +
combine when splitting) over resident device inputs.  Cold-HBM timing: the
KV pool is replicated into several device copies (>= 1 GiB together, more
than the 256 MB last-level cache) and the copies rotate per step.

Prints ONE JSON line.  `--gpus N` with N > 1 exits: this library runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
METRIC = "effective KV-cache read GB/s (% of MI355X HBM peak) + µs/decode step"


def _log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def make_case(name):
    """The named workload; a "_hm" suffix on a GQA workload stores the same
    cache with head-major pages [pages, Hkv, P, d]."""
    from decode_attention_paged_02_amd import workloads as W
    hm = 0
    if name.startswith("mla") and name.endswith("_qm"):   # the same case, queries on M
        name = name[:-3]
    if name.endswith("_hm") and name.startswith(("gqa", "ragged", "mqa")):
        name, hm = name[:-3], 1
    if name == "gqa_b64":
        return W.gqa_batch64(kv_layout=hm)
    if name == "gqa_b1_split":
        return W.gqa_long(1, kv_layout=hm)
    if name == "gqa_b4_split":
        return W.gqa_long(4, kv_layout=hm)
    if name == "mla_b16":
        return W.mla_b16()
    if name in ("ragged_fp8", "ragged_fp8_balanced"):
        return W.ragged_fp8(kv_layout=hm)
    if name == "gqa_b64_q2":
        return W.gqa_batch64_mtp(2, kv_layout=hm)
    if name == "mqa_b64_8k":
        return W.mqa_batch64_8k(kv_layout=hm)
    if name == "mla_b16_q2":
        return W.mla_b16_mtp(2)
    if name == "mla_b16_fp8":
        return W.mla_b16(kv_dtype="e4m3")
    if name == "mla_b16_320":
        return W.mla_b16(d_latent=256)
    raise SystemExit("unknown workload %s" % name)


CALL_KW = {"ragged_fp8": dict(num_splits=8, split_min_tokens=4096),
           # the balanced schedule (device-side chunking) on the same batch
           "ragged_fp8_balanced": dict(num_splits=8, schedule=1)}
GQA_WORKLOADS = ["gqa_b64", "gqa_b1_split", "gqa_b4_split", "ragged_fp8", "ragged_fp8_balanced",
                 "gqa_b64_q2", "mqa_b64_8k"]
MLA_WORKLOADS = ["mla_b16", "mla_b16_q2", "mla_b16_fp8", "mla_b16_320"]
# "_qm": the MLA kernel with the queries on the MFMA M dimension instead of the keys
WORKLOADS = GQA_WORKLOADS + [w + "_hm" for w in GQA_WORKLOADS] + MLA_WORKLOADS + [
    w + "_qm" for w in MLA_WORKLOADS]


def call_kw(workload):
    if workload.startswith("mla") and workload.endswith("_qm"):
        return dict(CALL_KW.get(workload[:-3], {}), variant=3)
    return dict(CALL_KW.get(workload[:-3] if workload.endswith("_hm") else workload, {}))


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, or None when it is missing or was taken on other sources of
    that kernel."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    from decode_attention_paged_02_amd.profiling import source_digest
    t = json.load(open(path))
    if t.get("source_digest") != source_digest(kernel):
        return None
    return t.get("bytes_per_launch")


def queue_ahead(cycles: int = 400_000):
    """Queue an idle kernel of `cycles` shader clocks (about 0.2 ms at
    2.4 GHz) on torch's current stream, the launch stream.  A timed region
    that starts right after a synchronize would otherwise also time the
    host's latency to launch its first step (about 30 us from Python, 1.5 us
    per step over 20 steps); behind this kernel the start event and the
    timed steps are already queued when the GPU reaches them, so the events
    time the steps alone."""
    import torch
    torch.cuda._sleep(cycles)


def run_gpu(case, workload, steps, warmup, pools, min_warmup_ms=100.0):
    import torch
    from decode_attention_paged_02_amd import accounting as A
    from decode_attention_paged_02_amd import pda

    dev = pda.to_device(case)
    kw = call_kw(workload)
    nbytes = A.case_kv_bytes(case)
    pool_bytes = dev.k_cache.numel() * dev.k_cache.element_size() * (1 if case.mla else 2)
    n_pools = max(pools, math.ceil((1 << 30) / max(pool_bytes, 1))) if pools > 0 else 1
    caches = [(dev.k_cache, dev.v_cache)]
    for _ in range(n_pools - 1):
        caches.append((dev.k_cache.clone(), None if dev.v_cache is None else dev.v_cache.clone()))
    o_shape, l_shape = pda._result_shapes(dev.q, case.head_dim_v)
    out = torch.empty(o_shape, dtype=dev.q.dtype, device="cuda")
    lse = torch.empty(l_shape, dtype=torch.float32, device="cuda")
    if case.mla:
        shape = pda.mla_shape(dev.q, dev.k_cache, dev.block_tables, head_dim_v=case.d_latent,
                              split_min_tokens=kw.get("split_min_tokens", 0),
                              causal=case.causal, schedule=kw.get("schedule", 0),
                              kv_scale=case.k_scale, variant=kw.get("variant", 0))
    else:
        shape = pda.gqa_shape(dev.q, dev.k_cache, dev.v_cache, dev.block_tables,
                              k_scale=case.k_scale, v_scale=case.v_scale,
                              split_min_tokens=kw.get("split_min_tokens", 0),
                              causal=case.causal, schedule=kw.get("schedule", 0),
                              kv_layout=case.kv_layout)
    nsplit = kw.get("num_splits", 0)
    plan = pda.plan(shape, mla=case.mla, num_splits=nsplit)
    ws = pda.workspace_for(shape, mla=case.mla, num_splits=nsplit, device="cuda")

    step = pda.PreparedCall(mla=case.mla, q=dev.q, caches=caches,
                            block_tables=dev.block_tables, context_lens=dev.context_lens,
                            scale=case.scale, out=out, lse=lse, shape=shape,
                            num_splits=nsplit, workspace=ws)

    # untimed warm-up: `warmup` steps, then more until at least min_warmup_ms
    # of GPU time has passed (the clocks settle during the first ~10 ms of
    # work after an idle period)
    w0 = torch.cuda.Event(enable_timing=True)
    w1 = torch.cuda.Event(enable_timing=True)
    w0.record()
    done = 0
    for i in range(warmup):
        step(i)
    done = warmup
    w1.record()
    torch.cuda.synchronize()
    warm_ms = w0.elapsed_time(w1)
    while warm_ms < min_warmup_ms:
        w1b = torch.cuda.Event(enable_timing=True)
        for i in range(50):
            step(done + i)
        done += 50
        w1b.record()
        torch.cuda.synchronize()
        warm_ms = w0.elapsed_time(w1b)
    # whole-job time over exactly `steps` back-to-back steps
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    queue_ahead()
    t0.record()
    for i in range(steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    # then the distribution of 100 single steps (each between its own events)
    n_dist = 100
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n_dist)]
    queue_ahead()
    for i, (e0, e1) in enumerate(ev):
        e0.record()
        step(steps + i)
        e1.record()
    torch.cuda.synchronize()
    each = sorted(e0.elapsed_time(e1) * 1000.0 for e0, e1 in ev)
    dist = {"steps": n_dist, "median": round(each[n_dist // 2], 3), "min": round(each[0], 3),
            "p90": round(each[min(n_dist - 1, (9 * n_dist) // 10)], 3)}
    return dict(total_ms=total_ms, kernel_us_mean=total_ms * 1000.0 / steps, step_us=dist,
                warmup_steps=done, warmup_ms=round(warm_ms, 2),
                overhead_bytes=A.case_overhead_bytes(case, plan.max_splits),
                kv_bytes=nbytes, n_pools=len(caches), max_splits=plan.max_splits,
                pages_per_split=plan.pages_per_split, workgroups=plan.workgroups,
                launches=(1 if plan.max_splits == 1 else 2) + (1 if plan.ordered else 0),
                probe=read_probe(case, dev, caches, shape, nsplit, steps) if not case.mla else None)


def read_probe(case, dev, caches, shape, num_splits, steps):
    """The streaming-read probe (pda_stream_probe) over the same pools: the
    K/V bytes of this call read with the attention kernels' access pattern
    and no arithmetic, on the GRID split layout of the same split count (1
    and 2 tiles in flight per wave; the faster counts).  Its time is the
    practical ceiling of that access pattern on this device."""
    import torch
    from decode_attention_paged_02_amd import pda
    sh = pda.Shape.from_buffer_copy(shape)
    sh.schedule = pda.PDA_SCHEDULE_GRID
    best = None
    for sd in (1, 2):
        pr = pda.StreamProbe(sh, caches, dev.block_tables, dev.context_lens,
                             num_splits=num_splits, steps_in_flight=sd)
        for i in range(200):
            pr(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        queue_ahead()
        e0.record()
        for i in range(steps):
            pr(i)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1000.0 / steps
        if best is None or us < best[0]:
            best = (us, sd)
    return {"us": round(best[0], 3), "steps_in_flight": best[1],
            "GB/s": round(A_kv_bytes(case) / (best[0] * 1e-6) / 1e9, 1)}


def A_kv_bytes(case):
    from decode_attention_paged_02_amd import accounting as A
    return A.case_kv_bytes(case)


APPEND_WORKLOADS = {"kv_append_b64": "gqa_b64", "kv_append_ragged_fp8": "ragged_fp8",
                    "kv_append_b64_hm": "gqa_b64_hm"}


def run_append(base: str, steps: int, warmup: int):
    """Time the KV append of one new token per sequence into the cache of an
    attention workload (f16 rows, or fp16 rows quantized into an fp8 cache):
    bytes = new rows read + cache rows written."""
    import numpy as np
    import torch
    from decode_attention_paged_02_amd import pda
    case = make_case(base)
    dev = pda.to_device(case)
    B, Hkv, d = case.batch, case.num_kv_heads, case.head_dim
    rng = np.random.default_rng(7)
    k_new = torch.from_numpy(rng.standard_normal((B, 1, Hkv, d)).astype(np.float16)).cuda()
    v_new = torch.from_numpy(rng.standard_normal((B, 1, Hkv, d)).astype(np.float16)).cuda()
    pos = (dev.context_lens - 1).contiguous()
    pda.paged_kv_append(k_new, v_new, dev.block_tables, pos, dev.k_cache, dev.v_cache,
                        k_scale=case.k_scale, v_scale=case.v_scale,
                        kv_layout=case.kv_layout)                       # validates the shapes
    # then the bare C call with marshalled arguments, so the host keeps ahead
    import ctypes
    shape = pda.make_shape(batch=B, num_q_heads=Hkv, num_kv_heads=Hkv, head_dim=d, head_dim_v=d,
                           page_size=case.page_size, max_pages_per_seq=case.max_pages,
                           num_pages=case.num_pages, q_dtype=pda.PDA_F16,
                           kv_dtype=pda._dtype_code(dev.k_cache, fp8_ok=True),
                           k_scale=case.k_scale, v_scale=case.v_scale, q_len=1,
                           kv_layout=case.kv_layout)
    args = [pda._ptr(t) for t in (k_new, v_new, dev.block_tables, pos, dev.k_cache, dev.v_cache)]
    args += [ctypes.byref(shape), pda._stream_handle(None)]
    lib = pda.load()

    def call():
        rc = lib.paged_kv_append(*args)
        if rc:
            raise pda.PdaError(rc, "paged_kv_append")

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    queue_ahead()
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / steps
    elem = {"f16": 2, "bf16": 2, "f32": 4, "e4m3": 1}[case.kv_dtype]
    nbytes = B * Hkv * 2 * d * (2 + elem)
    return {"us_per_step": round(us, 3), "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
            "bytes": nbytes, "cache_dtype": case.kv_dtype,
            "note": "HIP events around back-to-back calls; one token per sequence per step"}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(case, budget_s=20.0):
    """The fp64 oracle on the host over a bounded sample of the workload: the
    first whole sequences (all heads), timed at one thread and at every thread
    the oracle may use, each the median of 3 wall-clock runs.  The sample is
    sized per thread count so that the six runs take about budget_s together."""
    import statistics
    import numpy as np
    import oracle
    from decode_attention_paged_02_amd import accounting as A
    all_threads = oracle.max_threads()
    rows = np.zeros(case.q.shape[:-1], dtype=bool)     # [B, Hq] or [B, s_q, Hq]
    rows[0] = True
    t = time.perf_counter()
    _oracle_call(case, rows, 1)
    one_seq_1t = max(time.perf_counter() - t, 1e-4)    # one sequence on one thread
    per_run = budget_s / 6.0
    res = {}
    for threads in (1, all_threads):
        # whole sequences; with several threads, at least one per thread
        nseq = int(min(case.batch, max(1 if threads == 1 else threads,
                                       per_run * threads / one_seq_1t)))
        rows[:] = False
        rows[:nseq] = True
        times = []
        for _ in range(3):
            t = time.perf_counter()
            _oracle_call(case, rows, threads)
            times.append(time.perf_counter() - t)
        dt = statistics.median(times)
        nbytes = A.step_kv_bytes(case.context_lens[:nseq], num_kv_heads=case.num_kv_heads,
                                 head_dim=case.head_dim, head_dim_v=case.head_dim_v,
                                 kv_dtype=case.kv_dtype, mla=case.mla)
        res[threads] = dict(gbs=nbytes / dt / 1e9, nseq=nseq, median_s=dt,
                            us_step=dt * 1e6 * case.batch / nseq)
    top = res[all_threads]
    return {"value": round(top["gbs"], 4), "unit": "GB/s", "cores": all_threads,
            "kind": "oracle",
            "sample": "the first %d of %d sequences (all heads) of the timed workload, fp64 "
                      "oracle, median of 3 runs (%.2f s) on %d threads; one thread: the first "
                      "%d sequences, median %.2f s" % (
                          top["nseq"], case.batch, top["median_s"], all_threads,
                          res[1]["nseq"], res[1]["median_s"]),
            "one_thread": {"value": round(res[1]["gbs"], 5), "unit": "GB/s",
                           "us_per_step_equiv": round(res[1]["us_step"], 1)},
            "us_per_step_equiv": round(top["us_step"], 1),
            "host": {"cpu_model": _cpu_model(), "nproc": os.cpu_count(),
                     "affinity": len(os.sched_getaffinity(0))}}


def _oracle_call(case, rows, threads):
    import oracle
    if case.mla:
        return oracle.mla_attention(case.q, case.k_cache, case.block_tables, case.context_lens,
                                    scale=case.scale, d_latent=case.d_latent,
                                    q_dtype=case.q_dtype, kv_dtype=case.kv_dtype,
                                    kv_scale=case.k_scale, causal=case.causal, rows=rows,
                                    num_threads=threads)
    return oracle.paged_attention(case.q, case.k_cache, case.v_cache, case.block_tables,
                                  case.context_lens, scale=case.scale, q_dtype=case.q_dtype,
                                  kv_dtype=case.kv_dtype, k_scale=case.k_scale,
                                  v_scale=case.v_scale, causal=case.causal, rows=rows,
                                  kv_layout=case.kv_layout, num_threads=threads)


def bandwidth_probe(nbytes=2 << 30, reps=10):
    """Device-to-device copy bandwidth (bytes read + written) over nbytes
    buffers: a practical HBM figure next to the published peak."""
    import torch
    a = torch.empty(nbytes // 2, dtype=torch.float16, device="cuda").normal_()
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    queue_ahead()
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    r = {"copy_GBs": round(2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)}
    del a, b
    torch.cuda.empty_cache()
    return r


def summarize(r, steps):
    us_step = r["total_ms"] * 1000.0 / steps
    gbs = r["kv_bytes"] / (us_step * 1e-6) / 1e9
    kgbs = r["kv_bytes"] / (r["kernel_us_mean"] * 1e-6) / 1e9
    return us_step, gbs, kgbs


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500,
                    help="untimed steps first (the GPU reaches its steady clocks within ~10 ms)")
    ap.add_argument("--min-warmup-ms", type=float, default=100.0,
                    help="after --warmup steps, keep warming up until this much GPU time has "
                         "passed (untimed)")
    ap.add_argument("--workload", default="gqa_b64_hm", choices=WORKLOADS,
                    help="the timed workload (default: B=64 / ctx 1024 with head-major pages; "
                         "gqa_b64 is the same cache with token-major pages)")
    ap.add_argument("--pools", type=int, default=4, help="rotating KV pool copies (0: one, warm)")
    ap.add_argument("--others",
                    default="gqa_b64,gqa_b1_split_hm,gqa_b4_split_hm,mqa_b64_8k_hm,"
                            "ragged_fp8_balanced_hm,mla_b16,kv_append_b64_hm",
                    help="extra workloads measured into 'other_workloads' ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--no-bw-probe", action="store_true",
                    help="skip the device copy bandwidth probe")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this library runs on one GPU; multi-GPU runs are not supported "
              "(requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    from decode_attention_paged_02_amd import pda
    pda.load()

    _log("workload", args.workload)
    case = make_case(args.workload)
    r = run_gpu(case, args.workload, args.steps, args.warmup, args.pools, args.min_warmup_ms)
    us_step, gbs, kgbs = summarize(r, args.steps)
    kernel = "mla_mfma_kernel" if case.mla else "gqa_mfma_kernel"
    traffic = measured_traffic(args.workload, kernel)
    roof = {"bound": "hbm", "achieved": round(kgbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(kgbs / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": kernel,
            "launch_us_mean": round(r["kernel_us_mean"], 3),
            "launches_per_step": r["launches"],
            "timing": "HIP events on the launch stream around the timed region / steps",
            "step_definitions": {
                "us_per_step": "GPU time of the timed back-to-back steps (HIP events on the "
                               "launch stream around all of them) / steps; a ~0.2 ms idle "
                               "kernel queued ahead of the first event keeps the host's "
                               "launch latency out of the timed region",
                "step_us": "100 more steps, each between its own pair of events: median, min "
                           "and 90th percentile (per-step event overhead included)"},
            "algorithmic_bytes_per_launch": r["kv_bytes"],
            "step_us": r["step_us"], "overhead_bytes_per_step": r["overhead_bytes"]}
    if r.get("probe"):
        roof["read_probe"] = r["probe"]
        roof["frac_of_practical_ceiling"] = round(r["probe"]["us"] / us_step, 4)
    others = {}
    for w in [x for x in args.others.split(",") if x and x not in (args.workload, "none")]:
        _log("other workload", w)
        if w in APPEND_WORKLOADS:
            others[w] = run_append(APPEND_WORKLOADS[w], max(20, args.steps // 4), 5)
            continue
        c2 = make_case(w)
        st = max(20, args.steps // 4)
        r2 = run_gpu(c2, w, st, args.warmup, args.pools, args.min_warmup_ms)
        u2, g2, k2 = summarize(r2, st)
        others[w] = {"us_per_step": round(u2, 2), "GB/s": round(g2, 1),
                     "frac_of_peak": round(g2 / HBM_PEAK_GBS, 4),
                     "max_splits": r2["max_splits"], "kv_bytes": r2["kv_bytes"],
                     "step_us_median": r2["step_us"]["median"]}
        if r2.get("probe"):
            others[w]["read_probe_us"] = r2["probe"]["us"]
            others[w]["frac_of_practical_ceiling"] = round(r2["probe"]["us"] / u2, 4)
        del c2
    if not args.no_bw_probe:
        _log("bandwidth probe")
        roof["measured_device_bw"] = bandwidth_probe()
    # the read ceiling of the B=64 step per page layout (streaming probe)
    reads = {}
    if r.get("probe") and case.kv_layout == 1 and not case.mla:
        reads["head-major %s" % case.name] = r["probe"]["GB/s"]
    for w, o in others.items():
        if "read_probe_us" in o and w in ("gqa_b64", "gqa_b64_hm"):
            reads[("head-major " if w.endswith("_hm") else "token-major ") + w] = round(
                o["kv_bytes"] / (o["read_probe_us"] * 1e-6) / 1e9, 1)
    if reads:
        roof.setdefault("measured_device_bw", {})["read_probe_GBs"] = reads
    cpu = None
    if not args.no_cpu_baseline:
        _log("cpu baseline (oracle)")
        cpu = cpu_baseline(case, args.cpu_budget)
    dt = {"f16": "f16", "bf16": "bf16", "f32": "f32"}[case.q_dtype]
    if case.kv_dtype == "e4m3":
        dt = "e4m3 cache, " + dt
    line = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "warmup_done": {"steps": r["warmup_steps"], "gpu_ms": r["warmup_ms"]},
        "ms_per_step": round(us_step / 1000, 5),
        "us_per_step": round(us_step, 3), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dt,
        "data": "synthetic",
        "config": {"workload": case.name, "batch": case.batch,
                   "num_q_heads": case.num_q_heads, "num_kv_heads": case.num_kv_heads,
                   "head_dim": case.head_dim, "page_size": case.page_size,
                   "context_lens": "uniform %d" % int(case.context_lens[0])
                   if len(set(case.context_lens.tolist())) == 1 else "ragged",
                   "q_len": case.q_len,
                   "kv_layout": "head-major pages [pages, Hkv, P, d]" if case.kv_layout
                   else "token-major pages [pages, P, Hkv, d]",
                   "max_splits": r["max_splits"], "kv_bytes_per_step": r["kv_bytes"],
                   "rotating_pools": r["n_pools"]},
        "roofline": roof, "cpu_baseline": cpu, "other_workloads": others,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
