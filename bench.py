#!/usr/bin/env python3
"""Benchmark of the chunked-prefill hot path on one MI355X.

Step = one chunked prefill of a 4000-token GQA prompt (32 query / 8 KV
heads, head dim 128, bf16, cache bound at capacity 8192) in W = 512 chunks
through the C ABI: cpk_prefill_chunk per chunk (one launch each: chunk
attention that also appends the padded chunk's K/V to the cache, the
416-row tail padded to 512, truncation, true length recorded; the first
chunk, at past 0, starts the prompt over, so no separate length reset).  The step is captured once as a HIP graph and replayed
(checked bit for bit against an eager step); the eager per-call step time is
reported beside it.  Inputs are seeded synthetic N(0,1) values already
resident in HBM.

value  = algorithmic attention TFLOP/s of the whole step: 4*D*Hq flops per
         visible (query, key) pair, 131.10 GFLOP per step, / step time.
roofline = the attention kernel alone (each cpk_prefill_chunk launch):
         per-launch algorithmic flops over its average launch duration (HIP
         events on the launch stream), against the bf16 dense MFMA peak of
         2.5 PFLOP/s; the GPU's kernel timestamps of one profiled eager step
         give the kernel's name and a second average beside it.
secondary = the fp32 demo (time only); decode rows of the mixed-step
         workload (64 sequences, contexts uniform in [512, 16384]) as a
         decode-only packed step: KV bytes read per second against the 8 TB/s
         HBM peak, for the whole step and for the decode kernel alone; a
         steady-state W=512 chunk at past_len 7680; the same prompt chunked at
         W = 256, 512, 1024 and 2048; the ladder prompts (useful
         and issued TFLOP/s); the rolling fp16 cache against the larger of its
         HBM and MFMA bounds; the mixed decode + prefill step at budgets 2048
         and 8192 against its sum and max bounds.
cpu_baseline = the fp64 CPU oracle timed on this host on bounded samples of
         every workload (the headline figure: query rows of the GQA prompt in
         seeded random order), at all its threads and, for the demo and one
         GQA chunk, at one thread; same flop and byte accounting.

    python bench.py [--gpus 1] [--steps 400] [--warmup 100]
"""
import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bf16_w512_traffic.txt")
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_bf16_64seq_traffic.txt")
ATTN_SRC = os.path.join(ROOT, "chunked_prefill_causal_kv_amd", "csrc", "k_attn.hip")
DECODE_SRC = os.path.join(ROOT, "chunked_prefill_causal_kv_amd", "csrc", "k_decode.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def chunk_flops(past, real, Hq, D):
    """Algorithmic flops of one chunk: 4*D per visible (query, key) pair per
    query head; row i of the chunk sees past + i + 1 keys."""
    pairs = real * past + real * (real + 1) // 2
    return 4 * D * Hq * pairs


def src_sha(path=ATTN_SRC):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def attn_src_sha():
    return src_sha(ATTN_SRC)


def read_traffic(sha, path=TRAFFIC_FILE):
    """Measured HBM bytes per launch from a committed counter summary, or
    None if absent or taken on a different kernel source."""
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha") != sha:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def profile_kernels(torch, fn):
    """Kernel names, launch counts and average durations (us) of what fn
    runs, from the GPU's own kernel timestamps (torch.profiler over the ROCm
    tracer, the source rocprofv3 reads too).  None if the profiler is
    unavailable, or when an outside profiler (rocprofv3) already traces the
    process: two tracers in one process give wrong durations."""
    if any(k.startswith(("ROCPROF", "ROCP_")) for k in os.environ):
        return None
    try:
        from torch.profiler import ProfilerActivity, profile
        torch.cuda.synchronize()
        with profile(activities=[ProfilerActivity.CUDA]) as prof:
            fn()
            torch.cuda.synchronize()
        out = {}
        for e in prof.key_averages():
            total = getattr(e, "device_time_total", None)
            if total is None:
                total = getattr(e, "cuda_time_total", 0.0)
            if e.count and total:
                out[e.key] = (e.count, total / e.count)
        return out or None
    except Exception as exc:   # the profiler is optional instrumentation
        log(f"bench: kernel profiler unavailable ({exc})")
        return None


def pick_kernel_time(prof, *needles):
    """(name, launches, average us) of the profiled kernel whose name holds
    every needle and that ran the most launches, or None."""
    if not prof:
        return None
    cands = [(n, c, t) for n, (c, t) in prof.items() if all(x in n for x in needles)]
    return max(cands, key=lambda x: x[1]) if cands else None


# spin length (GPU clock cycles) that covers the host-side enqueue of one
# eight-chunk step
HOST_LEAD_CYCLES = 2_000_000


def bench_chunked(cpk, si, torch, steps, warmup):
    L, Hq, Hkv, D, W, CAP = 4000, 32, 8, 128, 512, 8192
    q, k, v = (x.cuda() for x in si.gqa_prompt(L=L, Hq=Hq, Hkv=Hkv, D=D))
    cache = cpk.KVCache(1, Hkv, CAP, D, torch.bfloat16)
    out = torch.empty_like(q)
    chunks = cpk.cpk_split_chunks(L, W)
    stream = torch.cuda.current_stream()
    flops = [chunk_flops(p, r, Hq, D) for p, r in chunks]

    def step(events):
        # each padded chunk is one launch of the attention kernel, which
        # also appends the chunk's K/V to the cache (fused append) and
        # records the slot's length; the first chunk (past 0) starts the
        # prompt over, so a pass needs no separate reset of the length
        for i, (past, rows) in enumerate(chunks):
            sl = slice(past, past + rows)
            if events is not None:
                events[i][0].record(stream)
            cpk.cpk_prefill_chunk(q[sl], k[sl], v[sl], cache, 0, past, W, pad=True, out=out[sl])
            if events is not None:
                events[i][1].record(stream)

    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        step(None)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # Per-launch durations: a spin kernel ahead of each step keeps the GPU
    # busy while the host enqueues the step's launches, so the GPU meets each
    # event pair with the kernel already queued between them and the events
    # bracket the kernel rather than the host's launch gaps.
    evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
            for _ in chunks] for _ in range(steps)]
    for s in range(steps):
        torch.cuda._sleep(HOST_LEAD_CYCLES)
        step(evs[s])
        torch.cuda.synchronize()
    per_chunk_ms = [[evs[s][i][0].elapsed_time(evs[s][i][1]) for s in range(steps)]
                    for i in range(len(chunks))]
    prof = profile_kernels(torch, lambda: step(None))
    ms_step = (t1 - t0) * 1e3 / steps
    total_flops = sum(flops)
    kern_ms = [sum(c) / len(c) for c in per_chunk_ms]
    achieved = (total_flops / len(chunks)) / (sum(kern_ms) / len(chunks) * 1e-3) / 1e12
    table = [{"past_len": p, "rows": r, "gflop": round(f / 1e9, 3),
              "ms": round(m, 4), "ms_median": round(statistics.median(c), 4),
              "ms_min": round(min(c), 4), "tflops": round(f / (m * 1e-3) / 1e12, 1)}
             for (p, r), f, m, c in zip(chunks, flops, kern_ms, per_chunk_ms)]
    attn = pick_kernel_time(prof, "attn_")
    return dict(ms_step=ms_step, total_flops=total_flops, achieved=achieved,
                kern_ms_avg=sum(kern_ms) / len(kern_ms), table=table, chunks=chunks,
                q=q, k=k, v=v, attn_kernel=attn)


def bench_step_graph(cpk, si, torch, steps, warmup, q, k, v):
    """The whole hot path for one prompt through the product entry point:
    cpk_prefill_chunk (append + attention, padded tail, length recorded) for
    every W=512 chunk.  Eight consecutive steps are captured once as a HIP
    graph and replayed (one step per graph when the step count is not a
    multiple of 8), so host launch gaps drop out and each replay's own
    launch cost (~7 us) is spread over its steps; every replay runs every
    kernel of every step.  Replays are checked bit for bit against an eager
    step, with eager work in between.  Returns ms per step."""
    L, Hkv, D, W, CAP = q.shape[0], 8, q.shape[2], 512, 8192
    cache = cpk.KVCache(1, Hkv, CAP, D, torch.bfloat16)
    out = torch.empty_like(q)
    chunks = cpk.cpk_split_chunks(L, W)

    def step():
        for past, rows in chunks:
            sl = slice(past, past + rows)
            cpk.cpk_prefill_chunk(q[sl], k[sl], v[sl], cache, 0, past, W, pad=True, out=out[sl])

    cache.lens[0] = 0
    step()
    torch.cuda.synchronize()
    ref_out, ref_k, ref_len = out.clone(), cache.k.clone(), cache.seqlens_k.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    per = 8 if steps % 8 == 0 else 1
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(per):
            step()
    torch.cuda.synchronize()
    for _ in range(3):
        out.zero_()
        cache.k.zero_()
        graph.replay()
        torch.cuda.synchronize()
        if not (torch.equal(out, ref_out) and torch.equal(cache.k, ref_k)
                and torch.equal(cache.seqlens_k, ref_len)):
            raise RuntimeError("graph replay differs from the eager step")
        step()
        torch.cuda.synchronize()
    for _ in range((warmup + per - 1) // per):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps // per):
        graph.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) * 1e3 / steps


def bench_demo_fp32(cpk, si, torch, reps=20):
    """The fp32 demo workload on the GPU: 1000 tokens, 8 heads, D 64, chunk
    256 (4 chunks: 256/256/256/232), unpadded, into an fp32 cache of
    capacity 1024; rewind + 4 cpk_prefill_chunk calls per pass.  A
    correctness workload: its time is reported, with no roofline target."""
    _, (q, k, v) = si.demo_qkv()
    q, k, v = (x.cuda() for x in (q, k, v))
    cache = cpk.KVCache(1, 8, 1024, 64, torch.float32)
    out = torch.empty_like(q)
    chunks = cpk.cpk_split_chunks(1000, 256)

    def run():
        if cache.lens[0]:
            cpk.cpk_rewind(cache, 0, 0)
        for past, rows in chunks:
            sl = slice(past, past + rows)
            cpk.cpk_prefill_chunk(q[sl], k[sl], v[sl], cache, 0, past, 256, pad=False, out=out[sl])

    for _ in range(3):
        run()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    f = 4 * 64 * 8 * sum(p + 1 for p in range(1000))
    return {"chunks": [list(c) for c in chunks], "gflop": round(f / 1e9, 3), "ms": round(ms, 4),
            "tflops": round(f / (ms * 1e-3) / 1e12, 2), "dtype": "fp32",
            "note": "eager calls (rewind + 4 chunk launches), HIP events over 20 passes"}


def bench_widths(cpk, si, torch, q, k, v, widths=(256, 512, 1024, 2048), reps=10, warm=3):
    """The 4000-token GQA prompt chunked at other widths W (the chunk-size
    trade-off of the pages: small chunks re-read the growing cache more
    often): rewind + cpk_prefill_chunk per chunk (padded tail), captured once
    as a HIP graph per W; median of reps replays after warm.  Each chunk
    launch takes the kernel the library picks for its size (W >= 1024: the
    128-column kernel).  TFLOP/s counts the prompt's causal pairs once."""
    L, Hq, Hkv, D = q.shape[0], q.shape[1], k.shape[1], q.shape[2]
    f = 4 * D * Hq * (L * (L + 1) // 2)
    table = {}
    for W in widths:
        cache = cpk.KVCache(1, Hkv, 8192, D, torch.bfloat16)
        out = torch.empty_like(q)
        chunks = cpk.cpk_split_chunks(L, W)

        def run():
            cpk.cpk_rewind(cache, 0, 0)
            for past, rows in chunks:
                sl = slice(past, past + rows)
                cpk.cpk_prefill_chunk(q[sl], k[sl], v[sl], cache, 0, past, W, pad=True,
                                      out=out[sl])

        cache.lens[0] = 0
        run()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        for _ in range(warm):
            graph.replay()
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        ms = statistics.median(times)
        table[f"W{W}"] = {"chunks": len(chunks), "ms": round(ms, 4),
                          "tflops": round(f / (ms * 1e-3) / 1e12, 1)}
    return {"prompt_tokens": L, "gflop": round(f / 1e9, 2), "per_width": table,
            "note": "rewind + padded cpk_prefill_chunk per chunk, graph-replayed, median of "
                    f"{reps} replays after {warm}"}


def bench_steady_chunk(cpk, si, torch, reps=200, warm=50):
    """One W=512 chunk at past_len 7680 (cache 8192): steady-state point,
    HIP events around reps back-to-back launches after warm ones."""
    Hq, Hkv, D, P, W = 32, 8, 128, 7680, 512
    cache = cpk.KVCache(1, Hkv, 8192, D, torch.bfloat16)
    si.fill_seeded(cache.k, 11)
    si.fill_seeded(cache.v, 12)
    q = si.randn((W, Hq, D), "bf16", si.generator(13)).cuda()
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    for _ in range(warm):
        cpk.cpk_chunk_attention(q, cache, 0, P, out=out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        cpk.cpk_chunk_attention(q, cache, 0, P, out=out)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    f = chunk_flops(P, W, Hq, D)
    return {"past_len": P, "rows": W, "gflop": round(f / 1e9, 2), "ms": round(ms, 4),
            "tflops": round(f / (ms * 1e-3) / 1e12, 1)}


def bench_decode(cpk, si, torch, reps=100, warm=20):
    """Decode rows of the mixed-step workload as a decode-only packed step."""
    Hq, Hkv, D, CAP = 32, 8, 128, 16400
    ctxs = si.mixed_contexts()
    n = len(ctxs)
    cache = cpk.KVCache(n, Hkv, CAP, D, torch.bfloat16)
    si.fill_seeded(cache.k, 21)
    si.fill_seeded(cache.v, 22)
    g = si.generator(23)
    q = si.randn((n, Hq, D), "bf16", g).cuda()
    kn = si.randn((n, Hkv, D), "bf16", g).cuda()
    vn = si.randn((n, Hkv, D), "bf16", g).cuda()
    slots = list(range(n))
    cu = list(range(n + 1))
    meta = torch.tensor(slots + cu + ctxs, dtype=torch.int32).cuda()
    max_ctx = max(ctxs) + 1
    ws = torch.empty(cpk.cpk_varlen_workspace_size(n, Hq, max_ctx, D) // 4 + 4,
                     dtype=torch.float32, device="cuda")
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    for _ in range(warm):
        cpk.cpk_varlen_step(q, kn, vn, cache, slots, cu, ctxs, out=out, ws=ws, dev_meta=meta)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        cpk.cpk_varlen_step(q, kn, vn, cache, slots, cu, ctxs, out=out, ws=ws, dev_meta=meta)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    kv_bytes = sum((c + 1) * Hkv * D * 2 * 2 for c in ctxs)
    io_bytes = n * Hq * D * 2 * 2 + n * Hkv * D * 2 * 2 * 2
    gbps = (kv_bytes + io_bytes) / (ms * 1e-3) / 1e9
    sha = src_sha(DECODE_SRC)
    prof = profile_kernels(torch, lambda: [cpk.cpk_varlen_step(q, kn, vn, cache, slots, cu, ctxs,
                                                               out=out, ws=ws, dev_meta=meta)
                                           for _ in range(reps)])
    dk = pick_kernel_time(prof, "decode_kernel")
    dc = pick_kernel_time(prof, "decode_combine")
    own = None
    if dk:
        kg = (kv_bytes + io_bytes) / (dk[2] * 1e-6) / 1e9
        own = {"bound": "hbm", "achieved": round(kg, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
               "frac": round(kg / PEAK_HBM_GBPS, 4), "kernel": dk[0][:90],
               "avg_us": round(dk[2], 2), "launches": dk[1],
               "combine_avg_us": round(dc[2], 2) if dc else None,
               "timer": "GPU kernel timestamps (torch.profiler over the ROCm tracer)"}
    return {"sequences": n, "kv_gb": round(kv_bytes / 1e9, 3), "ms": round(ms, 4),
            "GBps": round(gbps, 1), "frac_of_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4),
            "note": "whole packed step (split-KV decode with the new rows' append fused, "
                    "then the combine)",
            "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS,
                         "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4),
                         "traffic": read_traffic(sha, DECODE_TRAFFIC_FILE),
                         "kernel": "decode_kernel<bf16,128,4> + decode_combine (whole step)",
                         "timer": f"HIP events around {reps} back-to-back steps on the launch "
                                  f"stream after {warm}",
                         "kernel_source_sha": sha},
            "kernel_roofline": own}


def rolling_work(L, H, D, C, c, explicit_mask, elem=2):
    """(visible pairs, algorithmic bytes) of the rolling schedule: L tokens
    (a multiple of c) in chunks of c over a C-slot window.  Query row i of
    chunk j (position j*c + i) sees positions max(0, (j+1)*c - C) .. j*c + i.
    Bytes per chunk: q and out, the K/V of the keys in the window read once,
    the c new K/V rows written once, and the (c, C) mask when one is passed."""
    n = L // c
    pairs = sum(min(C, (j + 1) * c) * c - c * (c - 1) // 2 for j in range(n))
    row = H * D * elem
    nbytes = sum(2 * c * row + 2 * min(C, (j + 1) * c) * row + 2 * c * row +
                 (c * C * elem if explicit_mask else 0) for j in range(n))
    return pairs, nbytes


def issued_pairs(past, width):
    """(query, key) pairs of `width` rows at past: row i sees past + i + 1 keys."""
    return width * past + width * (width + 1) // 2


def bench_ladder(cpk, si, torch, reps=2, passes=10, warm=3):
    """Ladder workload: seven prompts (five seeded lengths, 1137, 1200), each
    prefilled twice on the same cache without clearing, through
    cpk_prefill_chunk with padding on.  Useful flops count real rows only,
    issued flops the padded widths.  ms is one pass over the workload, the
    average of `passes` timed passes after `warm` untimed ones."""
    Hq, Hkv, D, W, CAP = 32, 8, 128, 512, 8192
    lengths = si.ladder_prompt_lengths()
    prompts = [tuple(x.cuda() for x in si.gqa_prompt(L=L, seed=200 + i))
               for i, L in enumerate(lengths)]
    cache = cpk.KVCache(1, Hkv, CAP, D, torch.bfloat16)
    outs = [torch.empty_like(p[0]) for p in prompts]
    useful = issued = 0
    for L in lengths:
        for past, rows in cpk.cpk_split_chunks(L, W):
            useful += issued_pairs(past, rows)
            issued += issued_pairs(past, cpk.cpk_ladder_width(W, rows))

    def run():
        for (q, k, v), out, L in zip(prompts, outs, lengths):
            for _ in range(reps):
                if cache.lens[0]:
                    cpk.cpk_rewind(cache, 0, 0)
                for past, rows in cpk.cpk_split_chunks(L, W):
                    sl = slice(past, past + rows)
                    cpk.cpk_prefill_chunk(q[sl], k[sl], v[sl], cache, 0, past, W, pad=True,
                                          out=out[sl])

    for _ in range(warm):
        run()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(passes):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / passes
    # the same pass captured once as a HIP graph (host launch gaps drop out),
    # checked against the eager pass, then replayed
    ref = [o.clone() for o in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    for o, r in zip(outs, ref):
        if not torch.equal(o.view(torch.int16), r.view(torch.int16)):
            raise RuntimeError("ladder graph replay differs from the eager pass")
    e0.record(stream)
    for _ in range(passes):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    g_ms = e0.elapsed_time(e1) / passes
    f_useful = 4 * D * Hq * useful * reps
    f_issued = 4 * D * Hq * issued * reps
    return {"prompts": lengths, "runs_each": reps, "ms": round(ms, 3),
            "useful_gflop": round(f_useful / 1e9, 2), "issued_gflop": round(f_issued / 1e9, 2),
            "useful_tflops": round(f_useful / (ms * 1e-3) / 1e12, 1),
            "issued_tflops": round(f_issued / (ms * 1e-3) / 1e12, 1),
            "graph_ms": round(g_ms, 3),
            "graph_useful_tflops": round(f_useful / (g_ms * 1e-3) / 1e12, 1),
            "graph_issued_tflops": round(f_issued / (g_ms * 1e-3) / 1e12, 1),
            "note": "eager cpk_prefill_chunk calls (append + attention per chunk); graph_*: "
                    "the same pass captured as a HIP graph and replayed"}


def bench_rolling(cpk, si, torch, explicit_mask=True, ring=False, reps=50, warm=10,
                  deferred=False):
    """Rolling right-aligned cache: 4096 fp16 tokens, 16 heads, C = 2048,
    c = 256; per chunk roll_append (out of place, double-buffered: C rows
    moved) then roll_attention, or with ring=True one cpk_ring_step (the c
    new rows written into the ring by the attention launch); deferred=True
    takes the deferred form of either (cpk_roll_attention_deferred or
    cpk_ring_step_deferred: the chunk's key-range parts merged by the next
    chunk's launch, the last chunk's by one flush);
    with the explicit (c, C) additive mask (0 visible, -32768 masked) or
    visibility computed in the kernel.  Median of reps timed passes over the
    16 chunks."""
    L, H, D, C, c = 4096, 16, 128, 2048, 256
    q, k, v = (x.cuda() for x in si.rolling_inputs())
    n = L // c
    masks, pairs = [], 0
    rows = torch.arange(c, device="cuda").unsqueeze(1)
    slots = torch.arange(C, device="cuda").unsqueeze(0)
    for j in range(n):
        p = j * c + rows                       # absolute query positions
        a = (j + 1) * c - C + slots            # absolute position held by each slot
        vis = (a >= 0) & (a <= p)
        masks.append(torch.where(vis, 0.0, -32768.0).to(torch.float16).contiguous())
        pairs += int(vis.sum())
    assert pairs == rolling_work(L, H, D, C, c, explicit_mask)[0]
    bufs = [torch.zeros((1, H, C, D), dtype=torch.float16, device="cuda") for _ in range(4)]
    out = torch.empty_like(q)
    nws = cpk.cpk_roll_workspace_size(H, H, C, c, D, torch.float16)
    wss = [torch.empty(nws // 4 + 4, dtype=torch.float32, device="cuda") for _ in range(2)]

    def run():
        cur, start, pending = 0, 0, None
        for j in range(n):
            sl = slice(j * c, (j + 1) * c)
            m = masks[j] if explicit_mask else None
            if ring and deferred:
                pending, start = cpk.cpk_ring_step_deferred(
                    q[sl], k[sl], v[sl], bufs[0][0], bufs[1][0], (j + 1) * c, 0, start,
                    wss[j % 2], prev=pending, mask=m, out=out[sl])
                if j == n - 1:
                    cpk.cpk_roll_flush(pending)
                continue
            if ring:
                # the append runs inside the attention launch
                _, start = cpk.cpk_ring_step(q[sl], k[sl], v[sl], bufs[0][0], bufs[1][0],
                                             (j + 1) * c, 0, start, mask=m, out=out[sl])
                continue
            ko, vo = bufs[2 * cur], bufs[2 * cur + 1]
            kn, vn = bufs[2 * (1 - cur)], bufs[2 * (1 - cur) + 1]
            cpk.cpk_roll_append(ko, vo, k[sl].unsqueeze(0), v[sl].unsqueeze(0), kn, vn)
            cur = 1 - cur
            if deferred:
                pending = cpk.cpk_roll_attention_deferred(q[sl], kn[0], vn[0], (j + 1) * c, 0,
                                                          wss[j % 2], prev=pending, mask=m,
                                                          out=out[sl])
                if j == n - 1:
                    cpk.cpk_roll_flush(pending)
                continue
            cpk.cpk_roll_attention(q[sl], kn[0], vn[0], (j + 1) * c, 0, mask=m, out=out[sl])

    # the 16 chunks are captured once as a HIP graph (after an eager pass
    # that also allocates the split workspace), so host launch gaps drop out
    run()
    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    for _ in range(warm):
        graph.replay()
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), "replay differs"
    ms = statistics.median(times)
    f = 4 * D * H * pairs
    nbytes = rolling_work(L, H, D, C, c, explicit_mask)[1]
    t_hbm = nbytes / (PEAK_HBM_GBPS * 1e9) * 1e3
    t_mma = f / (PEAK_BF16_TFLOPS * 1e12) * 1e3
    if t_hbm >= t_mma:
        roof = {"bound": "hbm", "achieved": round(nbytes / (ms * 1e-3) / 1e9, 1),
                "peak": PEAK_HBM_GBPS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": round(f / (ms * 1e-3) / 1e12, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    roof.update({"frac": round(max(t_hbm, t_mma) / ms, 4), "algorithmic_bytes": nbytes,
                 "hbm_bound_ms": round(t_hbm, 4), "mfma_bound_ms": round(t_mma, 4),
                 "note": "whole 16-chunk schedule against the larger of its HBM and fp16 "
                         "MFMA bounds"})
    how = "the explicit (c, C) mask" if explicit_mask else "visibility computed in the kernel"
    what = ("ring_step_deferred (append fused into the attention, each chunk's split merged "
            "by the next chunk's launch, the last by a flush)" if ring and deferred else
            "ring_step (append fused into the attention)" if ring else
            "roll_append + roll_attention_deferred (each chunk's split merged by the next "
            "chunk's launch, the last by a flush)" if deferred else
            "roll_append + roll_attention")
    return {"chunks": n, "gflop": round(f / 1e9, 2), "ms": round(ms, 4), "ms_min": round(min(times), 4),
            "tflops": round(f / (ms * 1e-3) / 1e12, 1), "dtype": "fp16", "roofline": roof,
            "note": f"{what} with {how}, per chunk; 16 chunks replayed as a HIP graph, "
                    f"median of {reps} replays after {warm}"}


def bench_mixed(cpk, si, torch, budget, overlap=False, reps=10, paged=False, warm=3):
    """Mixed step: 64 running decodes (contexts U[512, 16384]) plus a
    20,000-token prompt under a token budget, one packed step per budget
    (packed inputs built before timing): cpk_varlen_step, or with
    overlap=True the decode rows and the prompt rows on two streams.  Each
    step is compared with sum = bytes/HBM + flops/MFMA and max = max of the
    two (perfect overlap).  The whole schedule is also captured as a HIP
    graph and replayed: its time per step is the inter-token latency proxy
    of the running decodes (one token each per step) and its total the
    time-to-first-token proxy of the prompt (ready after its last chunk).
    paged=True runs the same steps over a paged cache (256-position blocks,
    block table a seeded shuffle of the pool)."""
    Hq, Hkv, D, CAP, P = 32, 8, 128, 20480, 20000
    ctxs = si.mixed_contexts()
    n_dec = len(ctxs)
    if paged:
        bs = 256
        maxb = CAP // bs
        nb = (n_dec + 1) * maxb
        cache = cpk.PagedKVCache(n_dec + 1, Hkv, nb, bs, maxb, D, torch.bfloat16)
        perm = torch.randperm(nb, generator=si.generator(35))
        cache.block_table.copy_(perm.view(n_dec + 1, maxb).to(torch.int32))
    else:
        cache = cpk.KVCache(n_dec + 1, Hkv, CAP, D, torch.bfloat16)
    si.fill_seeded(cache.k, 31)
    si.fill_seeded(cache.v, 32)
    pq, pk, pv = (x.cuda() for x in si.gqa_prompt(L=P, seed=33))
    g = si.generator(34)
    steps, done, lens = [], 0, list(ctxs)
    while done < P:
        rows = cpk.cpk_plan_step(budget, n_dec, P - done)
        dq = si.randn((n_dec, Hq, D), "bf16", g).cuda()
        dk = si.randn((n_dec, Hkv, D), "bf16", g).cuda()
        dv = si.randn((n_dec, Hkv, D), "bf16", g).cuda()
        q = torch.cat([dq, pq[done:done + rows]])
        kn = torch.cat([dk, pk[done:done + rows]])
        vn = torch.cat([dv, pv[done:done + rows]])
        slots = list(range(n_dec + 1))
        cu = list(range(n_dec + 1)) + [n_dec + rows]
        past = lens + [done]
        meta = torch.tensor(slots + cu + past, dtype=torch.int32).cuda()
        ws = torch.empty(cpk.cpk_varlen_workspace_size(n_dec + 1, Hq, max(lens) + 1, D) // 4 + 4,
                         dtype=torch.float32, device="cuda")
        kv_bytes = sum((x + 1) * Hkv * D * 2 * 2 for x in lens) + (done + rows) * Hkv * D * 2 * 2
        flops = 4 * D * Hq * (issued_pairs(done, rows) + sum(x + 1 for x in lens))
        steps.append((q, kn, vn, slots, cu, past, meta, ws, torch.empty_like(q), kv_bytes, flops))
        lens = [x + 1 for x in lens]
        done += rows

    side = torch.cuda.Stream()

    def run(events=None):
        for i, (q, kn, vn, slots, cu, past, meta, ws, out, _, _) in enumerate(steps):
            if events is not None:
                events[i][0].record(torch.cuda.current_stream())
            if overlap:
                cpk.varlen_step_overlapped(q, kn, vn, cache, slots, cu, past, side, out=out,
                                           ws=ws, dev_meta=meta)
            else:
                cpk.cpk_varlen_step(q, kn, vn, cache, slots, cu, past, out=out, ws=ws,
                                    dev_meta=meta)
            if events is not None:
                events[i][1].record(torch.cuda.current_stream())

    run()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in steps]
    run(evs)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    ref_out = [st[8].clone() for st in steps]
    # the whole schedule as one graph (steps rewrite the same cache rows,
    # so replays are repeatable)
    cap_stream = torch.cuda.Stream()
    cap_stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap_stream):
        run()
    torch.cuda.current_stream().wait_stream(cap_stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for _ in range(warm):
        graph.replay()
    g_ms = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(torch.cuda.current_stream())
        graph.replay()
        e1.record(torch.cuda.current_stream())
        torch.cuda.synchronize()
        g_ms.append(e0.elapsed_time(e1))
    for st, ro in zip(steps, ref_out):
        assert torch.equal(st[8].view(torch.int16), ro.view(torch.int16)), "replay differs"
    g_tot = statistics.median(g_ms)
    table = []
    for (*_, kv_bytes, flops), m in zip(steps, ms):
        t_mem = kv_bytes / (PEAK_HBM_GBPS * 1e9) * 1e3
        t_mma = flops / (PEAK_BF16_TFLOPS * 1e12) * 1e3
        table.append({"ms": round(m, 4), "sum_bound_ms": round(t_mem + t_mma, 4),
                      "max_bound_ms": round(max(t_mem, t_mma), 4),
                      "tflops": round(flops / (m * 1e-3) / 1e12, 1)})
    tot = sum(ms)
    return {"budget": budget, "streams": 2 if overlap else 1, "paged": paged,
            "steps": len(steps),
            "ms_total": round(g_tot, 3), "ms_per_step": round(g_tot / len(steps), 4),
            "itl_proxy_ms": round(g_tot / len(steps), 4), "ttft_proxy_ms": round(g_tot, 3),
            "ms_total_eager_calls": round(tot, 3),
            "sum_bound_ms_total": round(sum(t["sum_bound_ms"] for t in table), 3),
            "max_bound_ms_total": round(sum(t["max_bound_ms"] for t in table), 3),
            "frac_of_max_bound": round(sum(t["max_bound_ms"] for t in table) / g_tot, 4),
            "frac_of_sum_bound": round(sum(t["sum_bound_ms"] for t in table) / g_tot, 4),
            "per_step_eager": table}


def calibrate_copy(cpk, torch, reps=3):
    """A plain copy of known size for scaling HBM counters: roll_append with
    c = 1 reads K and V caches of 32 heads x 16384 x 128 bf16 (2 x 128 MiB)
    and writes the same amount."""
    H, C, D = 32, 16384, 128
    bufs = [torch.ones((1, H, C, D), dtype=torch.bfloat16, device="cuda") for _ in range(4)]
    chunk = [torch.ones((1, 1, H, D), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    for _ in range(reps):
        cpk.cpk_roll_append(bufs[0], bufs[1], chunk[0], chunk[1], bufs[2], bufs[3])
    torch.cuda.synchronize()
    nbytes = 2 * H * C * D * 2
    log(f"calibration copy: {nbytes} bytes read and {nbytes} bytes written per launch")
    return nbytes


def _oracle_rows_sample(oracle, np, si, threads, budget_s):
    """fp64 oracle on rows of the 4000-token GQA prompt drawn in a seeded
    random order, in batches of 64, until about budget_s seconds of CPU work
    have been spent (whole passes repeat; the sample ends inside one)."""
    L, Hq, Hkv, D = 4000, 32, 8, 128
    q, k, v = si.gqa_prompt(L=L, Hq=Hq, Hkv=Hkv, D=D)
    qs, ks, vs = (si.storage(x) for x in (q, k, v))
    kk = oracle.widen(np.ascontiguousarray(ks.transpose(1, 0, 2)), oracle.BF16)
    vv = oracle.widen(np.ascontiguousarray(vs.transpose(1, 0, 2)), oracle.BF16)
    rows_all = np.random.default_rng(0).permutation(np.arange(0, L))
    done_rows, flops, t_total = 0, 0, 0.0
    oracle.set_num_threads(threads)
    while t_total < budget_s:
        start = done_rows % len(rows_all)
        rows = np.sort(rows_all[start:start + 64])
        qq = oracle.widen(np.ascontiguousarray(qs[rows]), oracle.BF16)
        t0 = time.perf_counter()
        oracle.attention(qq, kk, vv, np.zeros(len(rows), np.int32), rows.astype(np.int32),
                         1.0 / math.sqrt(D))
        t_total += time.perf_counter() - t0
        flops += sum(4 * D * Hq * (int(r) + 1) for r in rows)
        done_rows += len(rows)
    return {"value": round(flops / t_total / 1e12, 6), "unit": "TFLOP/s", "threads": threads,
            "seconds": round(t_total, 2),
            "sample": f"{done_rows} query rows ({done_rows / L:.2f} passes over the 4000 rows "
                      f"of the prompt, seeded random order), all 32 heads, causal over the "
                      f"cache"}


def cpu_baseline(si, budget_s=6.0):
    """The fp64 CPU oracle (as it stands) timed on this host on a bounded
    sample of every workload, at all of the oracle's OpenMP threads and, for
    the fp32 demo and one chunk of the GQA prompt, at one thread.  Each
    entry counts only the work of the rows it evaluates (same flop and byte
    accounting as the GPU figures).  The headline entry is the GQA prompt
    sample."""
    import numpy as np

    import oracle
    n_all = oracle.num_threads()
    table = {}

    def run_timed(fn, threads):
        oracle.set_num_threads(threads)
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    # workload 1: the fp32 demo in full (4 chunks of 256 over 1000 tokens)
    _, (dq, dk, dv) = si.demo_qkv()
    dq, dk, dv = (si.storage(x) for x in (dq, dk, dv))
    f_demo = 4 * 64 * 8 * sum(p + 1 for p in range(1000))
    for threads in (n_all, 1):
        t = run_timed(lambda: oracle.prefill_chunked(oracle.Cache(oracle.F32, 1, 8, 1024, 64), 0,
                                                     dq, dk, dv, 256), threads)
        table[f"demo_fp32_threads_{threads}"] = {
            "value": round(f_demo / t / 1e12, 6), "unit": "TFLOP/s", "threads": threads,
            "seconds": round(t, 3), "sample": "whole demo: 1000 tokens, 8 heads, D 64, W 256"}

    # workload 2: sampled rows at all threads (headline), and chunk 0 in
    # full at one thread
    head = _oracle_rows_sample(oracle, np, si, n_all, budget_s)
    table[f"gqa_w512_rows_threads_{n_all}"] = head
    q, k, v = si.gqa_prompt()
    qs, ks, vs = (si.storage(x) for x in (q, k, v))

    def chunk0():
        c = oracle.Cache(oracle.BF16, 1, 8, 8192, 128)
        c.append(0, ks[:512], vs[:512], 0)
        oracle.attend_from_cache(c, 0, qs[:512], 0)
    t = run_timed(chunk0, 1)
    f0 = 4 * 128 * 32 * (512 * 513 // 2)
    table["gqa_w512_chunk0_threads_1"] = {
        "value": round(f0 / t / 1e12, 6), "unit": "TFLOP/s", "threads": 1, "seconds": round(t, 3),
        "sample": "chunk 0 of the 4000-token prompt in full (append + 512 rows x 32 heads)"}

    # workload 3: the 1137-token ladder prompt, padded forwards as the
    # oracle runs them (every padded row attended, real rows kept)
    useful = sum(issued_pairs(p, r) for p, r in oracle.split_chunks(1137, 512))
    issued = sum(issued_pairs(p, oracle.ladder_width(512, r))
                 for p, r in oracle.split_chunks(1137, 512))
    t = run_timed(lambda: oracle.prefill_chunked_padded(
        oracle.Cache(oracle.BF16, 1, 8, 8192, 128), 0, qs[:1137], ks[:1137], vs[:1137], 512),
        n_all)
    table[f"ladder_1137_threads_{n_all}"] = {
        "value": round(4 * 128 * 32 * useful / t / 1e12, 6), "unit": "TFLOP/s (useful)",
        "issued_tflops": round(4 * 128 * 32 * issued / t / 1e12, 6), "threads": n_all,
        "seconds": round(t, 3), "sample": "the 1137-token prompt, W 512, ladder-padded forwards"}

    # workload 4: the rolling fp16 cache in full (16 chunks)
    rq, rk, rv = (si.storage(x) for x in si.rolling_inputs())
    t = run_timed(lambda: oracle.roll_prefill(rq, rk, rv, 2048, 256, oracle.F16), n_all)
    pairs = rolling_work(4096, 16, 128, 2048, 256, False)[0]
    table[f"rolling_fp16_threads_{n_all}"] = {
        "value": round(4 * 128 * 16 * pairs / t / 1e12, 6), "unit": "TFLOP/s", "threads": n_all,
        "seconds": round(t, 3),
        "sample": "4096 tokens, 16 heads, C 2048, c 256: roll + masked attention over C slots"}

    # workload 5: decode rows (8 of the 64 sequences, KV bytes per second)
    # and one budget-2048 mixed step (those 8 decode rows plus 128 sampled
    # rows of the first 1984 prompt rows)
    ctxs = si.mixed_contexts()[:8]
    cap = max(ctxs) + 1 + 1984
    g = si.generator(41)
    n = len(ctxs)
    dcache = oracle.Cache(oracle.BF16, n + 1, 8, cap, 128)
    for i, c in enumerate(ctxs):
        dcache.k[i, :, :c] = si.storage(si.randn((8, c, 128), "bf16", g))
        dcache.v[i, :, :c] = si.storage(si.randn((8, c, 128), "bf16", g))
        dcache.lens[i] = c
    dq_ = si.storage(si.randn((n, 32, 128), "bf16", g))
    dk_ = si.storage(si.randn((n, 8, 128), "bf16", g))
    dv_ = si.storage(si.randn((n, 8, 128), "bf16", g))
    seqs = [(i, c) for i, c in enumerate(ctxs)]
    t = run_timed(lambda: oracle.varlen_step(dcache, seqs, dq_, dk_, dv_, list(range(n + 1))),
                  n_all)
    kvb = sum((c + 1) * 8 * 128 * 2 * 2 for c in ctxs) + n * 32 * 128 * 2 * 2
    table[f"decode_rows_threads_{n_all}"] = {
        "value": round(kvb / t / 1e9, 4), "unit": "GB/s", "threads": n_all,
        "seconds": round(t, 3),
        "sample": f"8 of the 64 decode sequences (contexts {ctxs}), one row each"}
    pq, pk, pv = (si.storage(x) for x in si.gqa_prompt(L=1984, seed=33))
    mq = np.concatenate([dq_, pq])
    mk = np.concatenate([dk_, pk])
    mv = np.concatenate([dv_, pv])
    sel = np.sort(np.random.default_rng(1).choice(1984, 128, replace=False))
    seqs_m = [(i, c + 1) for i, c in enumerate(ctxs)] + [(n, 0)]
    t = run_timed(lambda: oracle.varlen_step(dcache, seqs_m, mq, mk, mv,
                                             list(range(n + 1)) + [n + 1984],
                                             rows_idx={n: sel}), n_all)
    f_mix = 4 * 128 * 32 * (sum(c + 2 for c in ctxs) + int(sum(int(r) + 1 for r in sel)))
    table[f"mixed_budget_2048_threads_{n_all}"] = {
        "value": round(f_mix / t / 1e12, 6), "unit": "TFLOP/s", "threads": n_all,
        "seconds": round(t, 3),
        "sample": "one budget-2048 step: 8 decode rows + 128 of the 1984 prompt rows at past 0 "
                  "(append of all 1992 rows included)"}
    oracle.set_num_threads(n_all)
    return {"value": head["value"], "unit": "TFLOP/s", "cores": n_all, "kind": "oracle",
            "sample": head["sample"] + f", fp64, {head['seconds']} s; per-workload entries in "
                      "per_config",
            "per_config": table}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 400 timed steps (~0.1 s) after 100 warm-up steps: a 20-step window
    # (~5 ms) reads ~13% lower, as the GPU is still ramping up
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--secondary", default="all",
                    help="comma list of secondary groups to run: demo, steady, widths, "
                         "decode, ladder, rolling, mixed (default all)")
    ap.add_argument("--rolling", default="all",
                    help="comma list of rolling schedules to run: shift_mask, shift_computed, "
                         "ring_mask, ring_computed, shift_deferred_mask, shift_deferred_computed, "
                         "ring_deferred_mask, ring_deferred_computed (default all)")
    ap.add_argument("--mixed", default="all",
                    help="comma list of mixed steps to run, as budget[_two_streams][_paged] "
                         "(default all five)")
    ap.add_argument("--calibrate", action="store_true",
                    help="also run a plain copy of known size (for counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by KV head or by sequence with no exchange inside "
              "attention, but this benchmark runs and reports a single MI355X)", file=sys.stderr)
        sys.exit(2)

    import torch

    import chunked_prefill_causal_kv_amd as cpk
    import synth_inputs as si

    torch.cuda.set_device(0)
    if args.calibrate:
        calibrate_copy(cpk, torch)
    log("bench: chunked prefill 4000 tokens, W=512, GQA 32/8, D=128, bf16")
    r = bench_chunked(cpk, si, torch, args.steps, args.warmup)
    log(f"bench: eager {r['ms_step']:.3f} ms/step, attention {r['achieved']:.1f} TFLOP/s")
    ms_graph = bench_step_graph(cpk, si, torch, args.steps, args.warmup, r["q"], r["k"], r["v"])
    log(f"bench: graph-replayed step {ms_graph:.3f} ms")
    secondary = {}
    groups = {"demo", "steady", "widths", "decode", "ladder", "rolling", "mixed"}
    if args.secondary != "all":
        groups = set(args.secondary.split(","))
    if not args.no_secondary:
        secondary["per_chunk"] = r["table"]
    if not args.no_secondary and "demo" in groups:
        secondary["demo_fp32"] = bench_demo_fp32(cpk, si, torch)
        log(f"bench: fp32 demo {secondary['demo_fp32']}")
    if not args.no_secondary and "steady" in groups:
        secondary["steady_chunk"] = bench_steady_chunk(cpk, si, torch)
        log(f"bench: steady chunk {secondary['steady_chunk']}")
    if not args.no_secondary and "widths" in groups:
        secondary["chunk_widths"] = bench_widths(cpk, si, torch, r["q"], r["k"], r["v"])
        log(f"bench: chunk widths {secondary['chunk_widths']}")
    if not args.no_secondary and "decode" in groups:
        secondary["decode_rows"] = bench_decode(cpk, si, torch)
        log(f"bench: decode {secondary['decode_rows']}")
    if not args.no_secondary and "ladder" in groups:
        secondary["ladder"] = bench_ladder(cpk, si, torch)
        log(f"bench: ladder {secondary['ladder']}")
    if not args.no_secondary and "rolling" in groups:
        variants = {"shift_mask": ("rolling_fp16", True, False, False),
                    "shift_computed": ("rolling_fp16_computed_mask", False, False, False),
                    "ring_mask": ("rolling_fp16_ring", True, True, False),
                    "ring_computed": ("rolling_fp16_ring_computed_mask", False, True, False),
                    "shift_deferred_mask": ("rolling_fp16_deferred", True, False, True),
                    "shift_deferred_computed": ("rolling_fp16_deferred_computed_mask", False,
                                                False, True),
                    "ring_deferred_mask": ("rolling_fp16_ring_deferred", True, True, True),
                    "ring_deferred_computed": ("rolling_fp16_ring_deferred_computed_mask", False,
                                               True, True)}
        names = list(variants) if args.rolling == "all" else args.rolling.split(",")
        for name in names:
            key, explicit, ring, deferred = variants[name]
            secondary[key] = bench_rolling(cpk, si, torch, explicit, ring=ring, deferred=deferred)
            log(f"bench: rolling {secondary[key]}")
    if not args.no_secondary and "mixed" in groups:
        for budget, overlap, paged in ((2048, False, False), (2048, True, False),
                                       (2048, False, True), (8192, False, False),
                                       (8192, True, False)):
            tag = f"{budget}" + ("_two_streams" if overlap else "") + ("_paged" if paged else "")
            if args.mixed != "all" and tag not in args.mixed.split(","):
                continue
            mixed = bench_mixed(cpk, si, torch, budget, overlap, paged=paged)
            key = f"mixed_budget_{tag}"
            secondary[key] = mixed
            log(f"bench: mixed budget {budget}, {mixed['streams']} stream(s)"
                f"{', paged' if paged else ''}: "
                f"{mixed['ms_per_step']} ms/step over {mixed['steps']} steps, TTFT proxy "
                f"{mixed['ttft_proxy_ms']} ms (bounds: sum {mixed['sum_bound_ms_total']} ms, "
                f"max {mixed['max_bound_ms_total']} ms in total)")
    sha = attn_src_sha()
    value = r["total_flops"] / (ms_graph * 1e-3) / 1e12
    line = {
        "metric": "chunk-attn TFLOP/s & % bf16 MFMA peak at W=512; decode-row KV GB/s",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_graph, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "GQA chunked prefill: 4000-token prompt in W=512 chunks "
                               "(7x512 + 416 padded to 512), 32 query / 8 KV heads, "
                               "head_dim 128, cache capacity 8192, seqlens_k",
                   "global_batch": 1, "seq_len": 4000, "chunk": 512, "parallelism": "none",
                   "step": "cpk_prefill_chunk per chunk; 8 steps captured per HIP "
                           "graph, replayed steps/8 times",
                   "ms_per_step_eager_calls": round(r["ms_step"], 4)},
        "roofline": {"bound": "mfma", "achieved": round(r["achieved"], 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(r["achieved"] / PEAK_BF16_TFLOPS, 4),
                     "traffic": read_traffic(sha),
                     "kernel": (r["attn_kernel"][0][:100] if r["attn_kernel"]
                                else "attention kernel of cpk_prefill_chunk"),
                     "avg_launch_ms": round(r["kern_ms_avg"], 4),
                     "timer": "HIP events bracketing each launch on its stream (a spin kernel "
                              "ahead of each step keeps the host's enqueue ahead), averaged "
                              "over the 8 chunk launches of each timed step",
                     "trace_avg_launch_ms": (round(r["attn_kernel"][2] * 1e-3, 4)
                                             if r["attn_kernel"] else None),
                     "trace_frac": (round(r["total_flops"] / len(r["chunks"]) /
                                          (r["attn_kernel"][2] * 1e-6) / 1e12 /
                                          PEAK_BF16_TFLOPS, 4) if r["attn_kernel"] else None),
                     "kernel_source_sha": sha},
        "secondary": secondary,
    }
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle on a bounded sample")
        line["cpu_baseline"] = cpu_baseline(si)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
