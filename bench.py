"""Paged decode benchmark on one MI355X.

A step is one fi_paged_decode call (block-table gather, q.K, online softmax,
P.V, fp32 partials and the fixed-order merge) over the whole Llama-3-8B-like
decode batch: 64 requests, 32 q / 8 kv heads, head_dim 128, page size 16,
kv_len ~ U[512, 4096], bf16 N(0,1) K/V in a randomly permuted page pool. The
plan (host) is built once per batch, as a serving step reuses it for every
layer; its host time is reported separately.

Prints one JSON line. ``value`` is the achieved KV throughput (algorithmic
K+V bytes over the measured time per call, inputs resident in HBM).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention µs/call and achieved KV HBM GB/s (% of peak), 1 GPU"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
CONFIG_INDEX = 1               # the Llama-3-8B-like decode batch
KERNEL_SOURCES = ("paged_kv_attention_amd/csrc/fi_attention.hip",
                  "paged_kv_attention_amd/csrc/fi_decode_body.h",
                  "paged_kv_attention_amd/csrc/fi_device.h",
                  "paged_kv_attention_amd/csrc/fi_internal.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_llama3_8b_decode.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w) -> dict:
    """Bytes a perfect kernel must move for one call: K and V of exactly
    kv_len tokens per request and kv head, q, o, lse and the page ids."""
    kv = w.kv_bytes()
    q = w.q.numel() * 2
    o = q
    lse = w.batch * w.num_qo_heads * 4
    idx = int(w.kv_indptr[-1]) * 4
    return dict(kv=kv, total=kv + q + o + lse + idx)


def _profile_summary():
    """The committed rocprofv3 summary of the headline kernel (HBM counters
    and kernel-trace duration), only if it was taken on the current kernel
    source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t


def measured_traffic(launches_bytes: float):
    """HBM traffic per launch from the committed rocprofv3 counter summary."""
    t = _profile_summary()
    return t.get("hbm_bytes_per_launch") if t else None


def traced_launch(total_bytes: float):
    """The kernel-trace average duration of the same kernel from the committed
    rocprofv3 summary, and the roofline fraction it gives."""
    t = _profile_summary()
    k = t.get("kernel_trace") if t else None
    if not k:
        return None
    return {"avg_launch_us": k["avg_us"],
            "frac": round(total_bytes / (k["avg_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "source": k["source"]}


def cpu_baseline(w, budget_s: float):
    """The fp64 oracle on the host cores over the same batch, repeated until
    about ``budget_s`` seconds of work are done."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    kp, vp = w.k_cache.float().numpy(), w.v_cache.float().numpy()
    q = w.q.double().numpy()
    args = (w.kv_indptr.numpy(), w.kv_indices.numpy(), w.kv_len.numpy(), w.page_size, w.sm_scale)
    # size the sample by KV tokens: time the first few requests, then take
    # requests in order (and whole-batch repeats) for about budget_s seconds
    lens = [int(x) for x in w.kv_len]
    probe = list(range(min(4, w.batch)))
    oracle.paged_decode(q, kp, vp, *args, requests=probe[:1])   # first-call costs
    t0 = time.perf_counter()
    oracle.paged_decode(q, kp, vp, *args, requests=probe)
    per_tok = (time.perf_counter() - t0) / max(1, sum(lens[r] for r in probe))
    n_req, toks = 0, 0
    while n_req < w.batch and (n_req == 0 or (toks + lens[n_req]) * per_tok <= budget_s):
        toks += lens[n_req]
        n_req += 1
    reps = max(1, int(budget_s / max(1e-9, toks * per_tok)))
    reqs = list(range(n_req))
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.paged_decode(q, kp, vp, *args, requests=reqs)
    dt = time.perf_counter() - t0
    per_tok = w.num_kv_heads * w.head_dim * 2 * 2
    kv = int(w.kv_len[:n_req].sum()) * per_tok * reps
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"value": kv / dt / 1e9, "unit": "GB/s", "cores": int(min(cores, blas_threads)),
            "kind": "oracle",
            "sample": f"fp64 NumPy oracle, first {n_req} of {w.batch} requests x {reps} repeat(s), "
                      f"{dt:.1f} s wall, KV bytes of the sample / wall time"}


def _pct(xs, q):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, max(0, int(round(q * (len(xs) - 1)))))]


def cold_us_per_call(step, dev, n=50):
    """Time of one call with nothing of its inputs cached: reading 1 GiB
    between calls evicts L2 and the 256 MB Infinity Cache (a read, so no
    dirty lines are left to be written back during the call); the scrub's own
    time is measured alone and subtracted. A serving step reads each layer's
    KV once, so this is the time a model sees; the plain loop re-reads the
    same KV and can hit the Infinity Cache when it fits."""
    import torch
    scrub = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)

    def loop(with_call):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            torch.sum(scrub, dim=0, out=sink)
            if with_call:
                step()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n
    loop(True)
    both = [loop(True) for _ in range(3)]
    alone = [loop(False) for _ in range(3)]
    del scrub
    return round(min(both) - min(alone), 2)


def graph_us_per_call(call, calls=10, replays=20):
    """Median per-call time of HIP-graph replays of ``calls`` back-to-back
    calls: the GPU's time per call without the host's launch cost."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(calls):
            call()
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    samples = []
    for _ in range(replays):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        e1.synchronize()
        samples.append(e0.elapsed_time(e1) * 1e3 / calls)
    del graph
    return round(_pct(samples, 0.5), 2)


def measure_variants(args, w, g, plan, step, dev):
    """Context for the main number, measured after the timed region:
    HIP-graph replays, cold-cache calls, and the deterministic-mode plan."""
    import torch
    import paged_kv_attention_amd as fi
    res = {}
    # (1) HIP graph of 10 calls, replayed; per-call time of each replay
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(10):
            step()
    for _ in range(5):
        graph.replay()
    torch.cuda.synchronize()
    samples = []
    for _ in range(max(10, args.steps // 10)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        e1.synchronize()
        samples.append(e0.elapsed_time(e1) * 1e3 / 10)
    res["graph_replay_us"] = {"replays": len(samples), "calls_per_replay": 10,
                              "median": round(_pct(samples, 0.5), 2),
                              "p10": round(_pct(samples, 0.1), 2),
                              "p90": round(_pct(samples, 0.9), 2)}
    del graph
    # (2) cold cache
    res["cold_us_per_call"] = cold_us_per_call(step, dev)
    # (3) deterministic-mode plan (chunks fixed per request) on the same batch
    dplan = fi.Plan("decode", w.kv_indptr, w.kv_len, w.num_qo_heads, w.num_kv_heads, w.head_dim,
                    w.page_size, device=dev, deterministic=True, engine=args.engine,
                    det_chunk_pages=args.det_chunk_pages)
    out = torch.empty_like(g.q)

    def dstep():
        fi.paged_decode(dplan, g.q, g.k_cache, g.v_cache, g.kv_indices, w.sm_scale, out=out)
    for _ in range(args.warmup):
        dstep()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        dstep()
    e1.record()
    torch.cuda.synchronize()
    res["deterministic_us_per_call"] = round(e0.elapsed_time(e1) * 1e3 / args.steps, 2)
    return res


def explore(args, dev):
    """Timing of one call on another configuration (decode, cascade or
    append), for the design notes; prints its own JSON line."""
    import torch
    import paged_kv_attention_amd as fi
    from workloads import CONFIG_NAMES, POD_MIX_NAME, make_config, make_pod_mix
    if args.pod_mix:
        w, name = make_pod_mix(poison=False), POD_MIX_NAME
    elif args.sparse_video:
        from workloads import SPARSE_VIDEO_NAME, make_sparse_video
        w, name = make_sparse_video(poison=False), SPARSE_VIDEO_NAME
    else:
        w, name = make_config(args.config, poison=False), CONFIG_NAMES[args.config]
    if args.kv != "bf16" and w.kind != "decode":
        raise SystemExit(f"bench.py: --kv {args.kv} applies to the decode configurations")
    if args.kv == "fp8":
        from workloads import to_fp8_cache
        w = to_fp8_cache(w, poison=False)
    elif args.kv == "mxfp4":
        from workloads import to_mxfp4_cache
        w = to_mxfp4_cache(w, poison=False)
    g = w.to(dev)
    kw = dict(deterministic=args.mode == "deterministic", workers_per_cu=args.workers_per_cu,
              min_chunk_pages=args.min_chunk_pages, det_chunk_pages=args.det_chunk_pages,
              engine=args.engine)
    if w.kind == "decode":
        plan = fi.Plan("decode", w.kv_indptr, w.kv_len, w.num_qo_heads, w.num_kv_heads,
                       w.head_dim, w.page_size, device=dev, kv_format=args.kv, merge=args.merge,
                       **kw)
        if args.kv == "fp8":
            call = lambda o, l: fi.paged_decode_fp8(plan, g.q, g.k_fp8, g.v_fp8, g.k_scale,  # noqa
                                                    g.v_scale, g.kv_indices, w.sm_scale,
                                                    out=o, lse=l)
        elif args.kv == "mxfp4":
            call = lambda o, l: fi.paged_decode_mxfp4(plan, g.q, g.k_fp4, g.v_fp4,  # noqa
                                                      g.k_bscale, g.v_bscale, g.kv_indices,
                                                      w.sm_scale, out=o, lse=l)
        else:
            call = lambda o, l: fi.paged_decode(plan, g.q, g.k_cache, g.v_cache,  # noqa
                                                g.kv_indices, w.sm_scale, out=o, lse=l)
        flops = 4 * w.head_dim * w.num_qo_heads * int(w.kv_len.sum())
    elif w.kind == "cascade":
        plan = fi.Plan("cascade", w.kv_indptr, w.kv_len, w.num_qo_heads, w.num_kv_heads,
                       w.head_dim, w.page_size, prefix_indptr=w.prefix_indptr,
                       prefix_len=w.prefix_len, req_prefix_group=w.req_prefix_group,
                       device=dev, launch=args.launch, pod_wide_blocks=args.pod_wide_blocks, **kw)
        call = lambda o, l: fi.cascade(plan, g.q, g.k_cache, g.v_cache,  # noqa
                                       g.prefix_indices, g.kv_indices, w.sm_scale, out=o, lse=l)
        per_req = w.kv_len.long() + w.prefix_len[0].long()
        flops = 4 * w.head_dim * w.num_qo_heads * int(per_req.sum())
    elif w.kind == "block_sparse":
        plan = fi.BlockSparsePlan(w.q.shape[0], int(w.kv_len[0]), w.row_block_sz,
                                  w.col_block_sz, w.block_mask, w.kv_indices, w.num_qo_heads,
                                  w.num_kv_heads, w.head_dim, w.page_size, device=dev,
                                  launch=args.launch, pod_wide_blocks=args.pod_wide_blocks,
                                  **{k: v for k, v in kw.items() if k != "engine"})
        call = lambda o, l: fi.block_sparse_attention(plan, g.q, g.k_cache,  # noqa
                                                      g.v_cache, w.sm_scale, out=o, lse=l)
        # attended (query, key) pairs, every q head: 4 D flops each
        G = w.num_qo_heads // w.num_kv_heads
        pairs = (w.block_mask.double() * w.row_block_sz[:, :, None].double()
                 * w.col_block_sz[:, None, :].double()).sum()
        flops = int(4 * w.head_dim * G * float(pairs))
    else:
        plan = fi.Plan("append", w.kv_indptr, w.kv_len, w.num_qo_heads, w.num_kv_heads,
                       w.head_dim, w.page_size, qo_indptr=w.qo_indptr, causal=True,
                       device=dev, launch=args.launch, pod_wide_blocks=args.pod_wide_blocks, **kw)
        call = lambda o, l: fi.paged_append(plan, g.q, g.k_cache, g.v_cache,  # noqa
                                            g.kv_indices, w.sm_scale, k_new=g.k_new,
                                            v_new=g.v_new, out=o, lse=l)
        qo = (w.qo_indptr[1:] - w.qo_indptr[:-1]).long()
        pre = w.kv_len.long() - qo
        flops = 4 * w.head_dim * w.num_qo_heads * int((qo * pre + qo * (qo + 1) // 2).sum())
    # outputs preallocated, as a serving loop holds them: the timed calls
    # allocate nothing
    T = g.q.shape[0]
    out = torch.empty_like(g.q)
    lse_buf = torch.empty(T, w.num_qo_heads, dtype=torch.float32, device=dev)
    raw_call = call
    call = lambda: raw_call(out, lse_buf)  # noqa: E731
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        call()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    graph_us = graph_us_per_call(call) if args.variants else None
    with fi.KernelTimer(args.steps) as kt:
        for _ in range(args.steps):
            call()
        torch.cuda.synchronize()
    kern_ms = kt.total_ms / max(1, kt.calls)
    cold_us = cold_us_per_call(call, dev) if args.variants else None
    kv = {"fp8": w.kv_bytes_fp8, "mxfp4": w.kv_bytes_mxfp4}.get(args.kv, w.kv_bytes)()
    extra = {}
    if w.kind != "decode":
        extra = {"launch": args.launch, "pod_wide_blocks": plan.info()["pod_wide_blocks"]}
    else:
        extra = {"merge": "fused" if plan.info()["fused_merge"] else "separate"}
    print(json.dumps({"workload": name, "mode": args.mode,
                      "engine": args.engine, "kv": args.kv, **extra,
                      "us_per_call": round(ms * 1e3, 2), "attention_us": round(kern_ms * 1e3, 2),
                      "graph_us_per_call": graph_us, "cold_us_per_call": cold_us,
                      "kv_bytes": kv, "kv_GBps": round(kv / ms / 1e6, 1),
                      "pct_hbm_peak": round(100 * kv / ms / 1e6 / HBM_PEAK_GBS, 2),
                      "flops": flops, "TFLOPs": round(flops / ms / 1e9, 1),
                      "pct_mfma_peak": round(100 * flops / ms / 1e9 / 2500.0, 2)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--mode", choices=("balanced", "deterministic"), default="balanced")
    ap.add_argument("--workers-per-cu", type=int, default=0)
    ap.add_argument("--min-chunk-pages", type=int, default=0)
    ap.add_argument("--det-chunk-pages", type=int, default=0,
                    help="deterministic mode: chunk size in pages (0 = the library default)")
    ap.add_argument("--engine", choices=("default", "mfma", "valu"), default="default",
                    help="units for the decode-style levels")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for cpu_baseline (0 = skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for counter scaling)")
    ap.add_argument("--kv", choices=("bf16", "fp8", "mxfp4"), default="bf16",
                    help="KV cache format for the exploratory decode lines (--config)")
    ap.add_argument("--no-variants", dest="variants", action="store_false",
                    help="skip the graph-replay, cold-cache and deterministic-mode context "
                         "(exploratory lines: the cold-cache time)")
    ap.add_argument("--config", type=int, default=CONFIG_INDEX,
                    help="other configurations print an exploratory line (not the bench line)")
    ap.add_argument("--explore", action="store_true",
                    help="print the exploratory line for the headline configuration too")
    ap.add_argument("--pod-mix", action="store_true",
                    help="exploratory line on the chunked-prefill mixed batch (64 decode "
                         "requests beside two 512-token prefill chunks)")
    ap.add_argument("--sparse-video", action="store_true",
                    help="exploratory line on the video-shaped variable block-sparse "
                         "self-attention (8192 tokens, 16 heads, 64 blocks per head)")
    ap.add_argument("--launch", choices=("default", "pod", "separate"), default="default",
                    help="append and cascade workloads: one POD launch for both kinds of rows, "
                         "or one launch per kind")
    ap.add_argument("--merge", choices=("default", "fused", "separate"), default="default",
                    help="decode: fold split units in the attention kernel (default) or in a "
                         "merge launch after it")
    ap.add_argument("--pod-wide-blocks", type=int, default=0,
                    help="POD launch: workgroups of the wide role (0 = the plan's choice)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the library runs on one GPU; --gpus must be 1 (sharding the path "
              "across GPUs is designed, not implemented).", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_attention_amd as fi
    from workloads import CONFIG_NAMES, make_config

    dev = torch.device("cuda:0")
    fi.load()
    if (args.config != CONFIG_INDEX or args.kv != "bf16" or args.pod_mix or args.sparse_video
            or args.explore):
        explore(args, dev)
        return
    print(f"bench: generating {CONFIG_NAMES[CONFIG_INDEX]}", file=sys.stderr, flush=True)
    w = make_config(CONFIG_INDEX, poison=False)
    g = w.to(dev)
    nbytes = algorithmic_bytes(w)

    plan_kw = dict(deterministic=args.mode == "deterministic",
                   workers_per_cu=args.workers_per_cu, min_chunk_pages=args.min_chunk_pages,
                   det_chunk_pages=args.det_chunk_pages, engine=args.engine, merge=args.merge)
    t0 = time.perf_counter()
    plan = fi.Plan("decode", w.kv_indptr, w.kv_len, w.num_qo_heads, w.num_kv_heads, w.head_dim,
                   w.page_size, device=dev, **plan_kw)
    torch.cuda.synchronize()
    plan_ms_first = (time.perf_counter() - t0) * 1e3
    # steady-state host plan time (re-plan into the same workspace)
    reps = 20
    t0 = time.perf_counter()
    for _ in range(reps):
        plan = fi.Plan("decode", w.kv_indptr, w.kv_len, w.num_qo_heads, w.num_kv_heads,
                       w.head_dim, w.page_size, device=dev, workspace=plan.workspace, **plan_kw)
    torch.cuda.synchronize()
    plan_us = (time.perf_counter() - t0) / reps * 1e6

    out = torch.empty_like(g.q)
    lse = torch.empty(w.batch, w.num_qo_heads, dtype=torch.float32, device=dev)

    def step():
        fi.paged_decode(plan, g.q, g.k_cache, g.v_cache, g.kv_indices, w.sm_scale, out=out,
                        lse=lse)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"bench: warmup done ({args.warmup} calls), timing {args.steps}", file=sys.stderr,
          flush=True)

    # Timed region: exactly `steps` calls, nothing else on the stream.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    ms_total = ev0.elapsed_time(ev1)
    ms_per_step = ms_total / args.steps
    # The attention kernel's own duration: the same calls again, each attention
    # launch recording a HIP event pair in its dispatch packet on its stream
    # (the start and end of the kernel's execution, as a kernel trace sees it).
    with fi.KernelTimer(args.steps) as kt:
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
    kern_ms = kt.total_ms / max(1, kt.calls)

    extra = measure_variants(args, w, g, plan, step, dev) if args.variants else None

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    gbs = nbytes["kv"] / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes["total"] / (kern_ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(nbytes["total"]),
            "kernel": "decode_kernel<128,2,false>", "algorithmic_bytes_per_launch": nbytes["total"],
            "avg_launch_us": round(kern_ms * 1e3, 2),
            "timing": "avg over a second pass of the same steps of each attention kernel's "
                      "execution, HIP events recorded in its dispatch (hipExtLaunchKernel) on "
                      "the launch stream",
            "rocprof": traced_launch(nbytes["total"])}
    res = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": CONFIG_NAMES[CONFIG_INDEX], "batch": w.batch,
                   "num_qo_heads": w.num_qo_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "page_size": w.page_size,
                   "kv_len": "uniform [512, 4096]", "seed": w.seed, "mode": args.mode, "engine": args.engine,
                   "kv_tokens": int(w.kv_len.sum())},
        "us_per_call": round(ms_per_step * 1e3, 2),
        "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "plan_host_us": round(plan_us, 1), "plan_first_ms": round(plan_ms_first, 2),
        "roofline": roof,
    }
    if extra:
        res["context"] = extra
    if args.cpu_budget > 0:
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
