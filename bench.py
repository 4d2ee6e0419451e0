#!/usr/bin/env python
"""Benchmark of the fused no-logits DSA indexer top-k on one MI355X.

One step = one idx_fused_topk call over the whole batch: threshold samples, thresholds,
fused score + filter into the candidate slab, slab select and the exact fallback.  The
default workload is the long-context prefill: 4096 rows x 1,048,576 keys (causal,
offset 1,044,480), 32 heads, head_dim 128, MXFP4 q/k, k = 2048.  Inputs are synthetic,
seeded, and resident in HBM before the timed region starts.

Prints exactly one JSON line on stdout; progress goes to stderr.

    python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--workload long|prefill|decode|tiny]
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

PEAK_TFLOPS = {"mxfp4": 10100.0, "e4m3": 5000.0}   # MI355X dense MFMA peaks
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = ["fused.hip", "score_core.hpp", "common.hpp"]

WORKLOADS = {
    "long": "long-context prefill: 4096 rows x 1,048,576 keys, causal offset 1,044,480, 32 heads, MXFP4, k=2048",
    "prefill": "prefill: 4096 rows x 65,536 keys, causal offset 61,440, 64 heads, e4m3 + per-key scale, k=2048",
    "decode": "decode/MTP: 128 requests x 4 rows, paged K (64-token pages), context 8K-256K, 64 heads, e4m3, k=2048",
    "tiny": "tiny: 64 rows x 4096 keys, 32 heads, integer e4m3, k=512",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "sparse_attention_indexer_score_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload, launch_bytes_alg):
    """HBM bytes of one fused score+filter launch from committed rocprofv3 counter runs,
    or None when they are missing or were taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"score_filter_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def cpu_threads():
    """Host threads for the CPU baseline: the process's CPU share, at most 16 (one GPU's share
    of a GPU machine)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(p, rows_sample):
    """The oracle as it stands, timed on the host cores over a bounded sample of rows: one
    oracle call (scores of the row's visible keys, then the full sort) per row, rows spread
    over a pool of threads, each running single-threaded BLAS (NumPy releases the GIL in the
    matmul and the sort).  One decode of K is included."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    threads = cpu_threads()
    t0 = time.perf_counter()
    with threadpool_limits(1):
        kd = oracle.all_keys(p) if p.page_table is None else None
        one = lambda r: oracle.select_topk(oracle.row_scores(p, r, kd_all=kd), p.topk)
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, rows_sample))
    dt = time.perf_counter() - t0
    pairs = int(sum(int(p.ke[r]) - int(p.ks[r]) for r in rows_sample))
    return {"value": pairs / dt / 1e9, "unit": "Gkey-scores/s", "cores": threads, "kind": "oracle",
            "host_cpus": os.cpu_count(),
            "sample": f"{len(rows_sample)} of {p.rows} rows (every {p.rows // len(rows_sample)}th), all their "
                      f"visible keys ({pairs} key-scores), scoring + full sort per row, rows over {threads} "
                      f"threads with single-threaded BLAS; includes one decode of K; {dt:.1f} s"}


def step_ms(fn, iters, flush=None):
    """Sorted per-call HIP-event times (ms) of fn() on torch's current stream (the stream the
    library launches on when given none); flush() runs before every call, outside its
    events."""
    import torch
    marks = []
    for _ in range(iters):
        if flush is not None:
            flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        marks.append((e0, e1))
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) for a, b in marks)


def graph_ms(fn, iters, flush=None):
    """Sorted per-replay HIP-event times (ms) of one call of fn() captured into a HIP graph
    (launch gaps between the call's kernels removed); flush() runs eagerly before every
    replay, outside its events.  The replays' results are those of an eager call (the library
    records kernel launches only)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    ms = step_ms(g.replay, iters, flush)
    del g
    return ms


def timed_ms(fn, iters, flush=None):
    """Median and minimum of step_ms."""
    ms = step_ms(fn, iters, flush)
    return ms[len(ms) // 2], ms[0]


def stage_pass(runner, iters, flush):
    """Per-stage HIP-event times of iters fused calls (recorded by the library on its launch
    stream), each preceded by the cache flush as in the timed steps: mean per stage."""
    import torch
    import sparse_attention_indexer_score_amd as sai
    sai.idx_timing_enable(iters)
    for _ in range(iters):
        flush()
        runner()
    torch.cuda.synchronize()
    rec = sai.idx_timing_read(iters)
    sai.idx_timing_disable()
    return {s: float(np.mean([c[s] for c in rec])) for s in sai.FUSED_STAGES}


def fused_leg(p, dev, iters, flush, what):
    """Fused top-k on one workload: cold per-call time (median, minimum), stage split and the
    score + filter kernel against the MFMA peak of the workload's format."""
    import torch
    import sparse_attention_indexer_score_amd as sai
    dp = sai.DeviceProblem.from_host(p, dev)
    runner = sai.FusedRunner(dp, p.topk)
    _, st = runner(stats=True)
    runner()
    torch.cuda.synchronize()
    ms = step_ms(runner, iters, flush)
    gms = graph_ms(runner, iters, flush)
    stages = stage_pass(runner, iters, flush)
    med = ms[len(ms) // 2]
    alg = p.pairs * 2 * 128 * p.heads
    k2 = stages["score_filter"]
    res = {"what": what, "ms": round(med, 4), "min_ms": round(ms[0], 4),
           "Gkey_scores_per_s": round(p.pairs / (med * 1e-3) / 1e9, 2),
           "score_filter_ms": round(k2, 4), "score_filter_TFLOPs": round(alg / (k2 * 1e-3) / 1e12, 1),
           "score_filter_frac": round(alg / (k2 * 1e-3) / 1e12 / PEAK_TFLOPS[p.fmt], 4),
           "peak_TFLOPs": PEAK_TFLOPS[p.fmt], "stage_ms": {s: round(v, 4) for s, v in stages.items()},
           "fallback_rows": st["fallback_rows"],
           "graph_ms": round(gms[len(gms) // 2], 4), "graph_min_ms": round(gms[0], 4)}
    del runner, dp
    torch.cuda.empty_cache()
    return res


def secondary_legs(dev, iters=20, main_workload="long"):
    """Measured beside the headline: the fused top-k on the other two fused workloads
    (long / prefill / decode), selection (HBM-bound) and materialised scoring: idx_select on
    the selection workload (64 rows, pitch 131072) and on the prefill workload's materialised
    scores (4096 x 65536 fp32, 1.04 GB), idx_score on prefill, and the consumer,
    idx_sparse_attn (512 rows x 2048 selected slots; HBM-bound gather).  Cold numbers flush L2
    and the 256 MB MALL with a 512 MiB fill before every call."""
    import torch
    import sparse_attention_indexer_score_amd as sai
    from sparse_attention_indexer_score_amd import workloads as wl
    flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    flush = lambda: flush_buf.fill_(0x5A)
    res = {}

    for w in ("long", "prefill", "decode"):
        if w == main_workload:
            continue
        log(f"[bench] fused top-k on the {w} workload")
        res[f"fused_{w}"] = fused_leg(wl.make(w), dev, iters, flush, WORKLOADS[w])
        log(f"[bench] fused {w}: {res[f'fused_{w}']['ms']} ms, K2 {res[f'fused_{w}']['score_filter_frac']} of peak")

    sp = wl.make("select")
    x = torch.from_numpy(sp.x).to(dev)
    length = torch.from_numpy(sp.length).to(dev)
    run = sai.SelectRunner(x, length, sp.topk)
    run()
    torch.cuda.synchronize()
    nbytes = int(sp.length.astype(np.int64).sum()) * 4 + x.shape[0] * sp.topk * 4
    cold, cold_min = timed_ms(run, iters, flush)
    warm, warm_min = timed_ms(run, iters)
    res["select_workload"] = {
        "what": "idx_select, 64 rows x pitch 131072, lengths U[2048, 131072], k=2048 (row split g=4)",
        "bytes": nbytes, "cold_ms": round(cold, 4), "cold_min_ms": round(cold_min, 4),
        "warm_ms": round(warm, 4), "cold_GBps": round(nbytes / (cold * 1e-3) / 1e9, 1),
        "warm_GBps": round(nbytes / (warm * 1e-3) / 1e9, 1)}
    log(f"[bench] select workload: cold {cold:.4f} ms, warm {warm:.4f} ms")
    del x, length, run

    pp = wl.make("prefill")
    dpp = sai.DeviceProblem.from_host(pp, dev)
    sr = sai.ScoreRunner(dpp, ld=int((pp.ke - pp.ks).max()))
    sr()
    torch.cuda.synchronize()
    s_med, s_min = timed_ms(sr, min(10, iters))
    pairs = pp.pairs
    res["score_prefill"] = {
        "what": "idx_score, prefill workload (4096 x 65536, e4m3, 64 heads): fp32 scores written",
        "ms": round(s_med, 4), "min_ms": round(s_min, 4), "Gkey_scores_per_s": round(pairs / (s_med * 1e-3) / 1e9, 2),
        "mfma_TFLOPs": round(pairs * 2 * 128 * pp.heads / (s_med * 1e-3) / 1e12, 1),
        "write_GBps": round(pairs * 4 / (s_med * 1e-3) / 1e9, 1)}
    log(f"[bench] idx_score prefill: {s_med:.4f} ms")
    vlen = (dpp.ke - dpp.ks).to(torch.int32)
    sel = sai.SelectRunner(sr.out, vlen, pp.topk)
    sel()
    torch.cuda.synchronize()
    nbytes = int(pairs) * 4 + pp.rows * pp.topk * 4
    cold, cold_min = timed_ms(sel, iters, flush)
    res["select_prefill_materialised"] = {
        "what": "idx_select over the prefill workload's materialised scores (4096 rows, 260,048,896 scores, k=2048)",
        "bytes": nbytes, "cold_ms": round(cold, 4), "cold_min_ms": round(cold_min, 4),
        "cold_GBps": round(nbytes / (cold * 1e-3) / 1e9, 1),
        "hbm_frac": round(nbytes / (cold * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    log(f"[bench] select over materialised prefill scores: cold {cold:.4f} ms")
    del sel, sr, dpp
    torch.cuda.empty_cache()

    # The consumer: sparse attention of 512 decode rows over their 2048 selected slots.
    a = wl.make("sparse_attn")
    q = torch.from_numpy(a.q.view(np.int16)).to(dev)
    kc, vc = torch.from_numpy(a.k_cache).to(dev), torch.from_numpy(a.v_cache).to(dev)
    sl = torch.from_numpy(a.slots).to(dev)
    out = torch.empty((a.rows, a.q.shape[1], 128), dtype=torch.float32, device=dev)
    att = lambda: sai.idx_sparse_attn(q, kc, vc, sl, a.softmax_scale, a.output_scale, out=out)
    att()
    torch.cuda.synchronize()
    hkv = a.k_cache.shape[1]
    valid = int(((a.slots >= 0) & (a.slots < a.k_cache.shape[0])).sum())
    nbytes = valid * hkv * 2 * 128 + a.slots.size * 4 + a.q.size * 2 + out.numel() * 4
    cold, cold_min = timed_ms(att, iters, flush)
    res["sparse_attn"] = {
        "what": f"idx_sparse_attn, {a.rows} rows x {a.slots.shape[1]} selected slots, {a.q.shape[1]} query / {hkv} KV "
                f"heads, head_dim 128, e4m3 KV cache of {a.k_cache.shape[0]} slots",
        "bytes": nbytes, "cold_ms": round(cold, 4), "cold_min_ms": round(cold_min, 4),
        "cold_GBps": round(nbytes / (cold * 1e-3) / 1e9, 1),
        "hbm_frac": round(nbytes / (cold * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    log(f"[bench] sparse attention: cold {cold:.4f} ms")
    del q, kc, vc, sl, out, flush_buf
    torch.cuda.empty_cache()
    return res


def flush_cold(dev):
    """A 512 MiB fill that evicts L2 and the MALL (the flush between cold calls)."""
    import torch
    buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    return lambda: buf.fill_(0x5A)


def dense_runner(dp, p):
    """The dense route: idx_score writes every visible score as fp32 [rows, max V], then
    idx_select reads them back (preallocated buffers, nothing allocated per call)."""
    import torch
    import sparse_attention_indexer_score_amd as sai
    sr = sai.ScoreRunner(dp, ld=int((p.ke - p.ks).max()))
    sel = sai.SelectRunner(sr.out, (dp.ke - dp.ks).to(torch.int32), p.topk)
    return (lambda: (sr(), sel())), sr, sel


def dense_leg(p, dp, dev, iters, flush, fused_ms):
    """Dense route on the given problem (cold calls, median and minimum) against the fused
    median: the logits the fused path never writes are written and read back here."""
    import torch
    run, sr, sel = dense_runner(dp, p)
    run()
    torch.cuda.synchronize()
    med, mn = timed_ms(run, iters, flush)
    res = {"what": "dense route on the same problem: idx_score writes fp32 [rows, max V], idx_select reads it",
           "ms": round(med, 4), "min_ms": round(mn, 4), "logits_bytes": int(p.pairs) * 4,
           "fused_ms": round(fused_ms, 4), "fused_over_dense_speedup": round(med / fused_ms, 3)}
    del run, sr, sel
    torch.cuda.empty_cache()
    return res


ROUTING = {
    # family: (generator, rows list, key counts)
    "prefill_e4m3_64h": ("prefill", (512, 2048, 4096), (4096, 8192, 16384, 32768, 65536, 131072)),
    "long_mxfp4_32h": ("long", (512, 2048, 4096), (16384, 65536, 262144, 1048576)),
}


def routing_table(dev, families=None, k=2048, iters=5):
    """Dense route (idx_score + idx_select) against the fused top-k per format, batch and
    context length (causal rows, every call cold), and the crossover per batch: the shortest
    context at which the fused path is faster."""
    import torch
    import sparse_attention_indexer_score_amd as sai
    from sparse_attention_indexer_score_amd import workloads as wl
    flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    flush = lambda: flush_buf.fill_(0x5A)
    table, crossover = [], {}
    for fam in (families or ROUTING):
        gen, rows_list, keys_list = ROUTING[fam]
        for rows in rows_list:
            cross = None
            for n in keys_list:
                if n < rows:
                    continue
                p = wl.make(gen, rows=rows, num_keys=n, topk=k)
                dp = sai.DeviceProblem.from_host(p, dev)
                fused = sai.FusedRunner(dp, k)
                fused()
                torch.cuda.synchronize()
                f_ms, _ = timed_ms(fused, iters, flush)
                d = dense_leg(p, dp, dev, iters, flush, f_ms)
                rec = {"family": fam, "rows": rows, "keys": n, "pairs": int(p.pairs), "fused_ms": round(f_ms, 4),
                       "dense_ms": d["ms"], "fused_over_dense_speedup": d["fused_over_dense_speedup"]}
                log(f"[routing] {rec}")
                table.append(rec)
                if cross is None and d["fused_over_dense_speedup"] > 1.0:
                    cross = n
                del fused, dp, p
                torch.cuda.empty_cache()
            crossover[f"{fam}/rows={rows}"] = cross
    return table, crossover


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-rows", type=int, default=512, help="rows in the oracle's timed sample (0: skip)")
    ap.add_argument("--routing", action="store_true",
                    help="only measure dense (idx_score + idx_select) against fused top-k over context lengths")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the selection and materialised-score measurements")
    ap.add_argument("--secondary-iters", type=int, default=20,
                    help="timed calls per secondary leg (fewer for profiler runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy (reference kernel for HBM counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: there is no multi-GPU path (rows would shard across GPUs "
              "with no communication). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_attention_indexer_score_amd as sai
    from sparse_attention_indexer_score_amd import workloads as wl

    if args.routing:
        dev = torch.device("cuda:0")
        torch.cuda.set_device(dev)
        table, crossover = routing_table(dev)
        print(json.dumps({"metric": "fused vs dense indexer top-k ms by format, batch and context length (causal, "
                                    "k=2048, every call cold), 1 GPU", "n_gpus": 1, "data": "synthetic",
                          "higher_is_better": False, "table": table,
                          "crossover_keys": crossover}), flush=True)
        return

    log(f"[bench] generating workload '{args.workload}'")
    t = time.perf_counter()
    p = wl.make(args.workload)
    log(f"[bench] generated in {time.perf_counter() - t:.1f}s: rows={p.rows} pairs={p.pairs}")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dp = sai.DeviceProblem.from_host(p, dev)
    k = p.topk
    runner = sai.FusedRunner(dp, k)
    torch.cuda.synchronize()
    log(f"[bench] resident; workspace {runner.nbytes / 2**20:.0f} MiB")

    if args.copy_calibration:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
        log("[bench] copy calibration kernel done (1 GiB read + 1 GiB write)")

    _, st = runner(stats=True)
    torch.cuda.synchronize()
    log(f"[bench] route: {st}")
    for _ in range(max(0, args.warmup - 1)):
        runner()
    torch.cuda.synchronize()

    # Timed steps: before each, a 512 MiB fill evicts the inputs from L2 and the 256 MB MALL
    # (outside the step's events); each step is bracketed by HIP events on the launch stream.
    flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    flush = lambda: flush_buf.fill_(0x5A)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms_steps = step_ms(runner, args.steps, flush)
    wall = time.perf_counter() - t0
    ms = ms_steps[len(ms_steps) // 2]
    log(f"[bench] {args.steps} steps: median {ms:.3f} ms, min {ms_steps[0]:.3f} ms, mean "
        f"{float(np.mean(ms_steps)):.3f} ms (wall {wall * 1e3 / args.steps:.3f} ms/step incl. flushes)")
    warm_ms = float(np.mean(step_ms(runner, args.steps)))
    # The same call captured into a HIP graph and replayed (flushed the same way).
    g_steps = graph_ms(runner, args.steps, flush)
    log(f"[bench] graph replays: median {g_steps[len(g_steps) // 2]:.3f} ms, min {g_steps[0]:.3f} ms")
    # Stage split from a separate pass of the same flushed steps (the library's own events on
    # its launch stream), so that the timed steps record nothing but their own two events.
    stage_ms = stage_pass(runner, args.steps, flush)
    log(f"[bench] stages: {stage_ms}")

    pairs = p.pairs
    value = pairs / (ms * 1e-3) / 1e9
    flops_per_pair = 2 * 128 * p.heads
    alg_flops = pairs * flops_per_pair                    # one fused score+filter launch
    k2_ms = stage_ms["score_filter"]
    achieved = alg_flops / (k2_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[p.fmt]
    traffic = load_traffic(args.workload, None)
    del flush_buf

    secondary = None
    if not args.no_secondary:
        dense = dense_leg(p, dp, dev, min(5, args.steps), flush_cold(dev), ms)
        log(f"[bench] dense route on the same problem: {dense['ms']} ms (fused {ms:.3f} ms)")
        secondary = {"dense_route": dense}
        secondary.update(secondary_legs(dev, iters=args.secondary_iters, main_workload=args.workload))

    cpu = None
    if args.cpu_rows > 0:
        step = max(1, p.rows // args.cpu_rows)
        rows_sample = list(range(0, p.rows, step))[:args.cpu_rows]
        log(f"[bench] timing the CPU oracle on {len(rows_sample)} rows")
        cpu = cpu_baseline(p, rows_sample)
        log(f"[bench] cpu baseline {cpu['value']:.5f} Gkey-scores/s on {cpu['cores']} threads")

    line = {
        "metric": "indexer Gkey-scores/s + fused top-k ms (4096 rows x 1M keys, k=2048), 1 GPU",
        "value": round(value, 3),
        "unit": "Gkey-scores/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "fused_topk_ms": round(ms, 4),
        "fused_topk_min_ms": round(ms_steps[0], 4),
        "fused_topk_warm_ms": round(warm_ms, 4),
        "fused_topk_graph_ms": round(g_steps[len(g_steps) // 2], 4),
        "timing": "median of the timed steps, each cold (L2 and MALL flushed by a 512 MiB fill before it); "
                  "fused_topk_graph_ms: the same call captured into a HIP graph and replayed, flushed the same way",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.fmt,
        "data": "synthetic",
        "config": {"workload": WORKLOADS[args.workload], "rows": p.rows, "key_scores": pairs, "k": k,
                   "heads": p.heads, "head_dim": 128, "format": p.fmt},
        "roofline": {"bound": "mfma", "kernel": "score_tiles_kernel<MXFP4|e4m3, H, FILTER> (fused score + filter)",
                     "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "alg_flops_per_launch": alg_flops, "launch_ms": round(k2_ms, 4)},
        "stage_ms": {s: round(v, 4) for s, v in stage_ms.items()},
        "route": {kk: st[kk] for kk in ("rows_store_all", "rows_sampled", "fallback_rows", "max_count",
                                         "min_count", "total_count", "cap", "sample_stride")},
        "logits_bytes_avoided": int(pairs) * 4 * 2,
        "secondary": secondary,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
