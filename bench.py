"""Indexer benchmark on one MI355X: keys scored per second for one whole indexer step
(logits over every cached key, causal masks, per-row top-k) on a seeded synthetic
workload, with the dominant kernel's roofline fraction and the CPU oracle beside it.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config 2] [--no-cpu-baseline]

Default workload: paged fp8 decode, 32 sequences, context lengths U[1024, 16384], 64
heads, logits width 32768, top-2048. ``--config 1..5`` selects one of the five
workloads. Inputs live in HBM before timing starts. Each timed step reads a different
copy of the K cache (copies totalling more than 512 MB rotate), so the 256 MB
Infinity Cache cannot hold a step's keys from the previous visit.

Prints ONE JSON line.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
FP8_MFMA_PEAK_TFLOPS = 5000.0  # MI355X dense fp8, published
FP4_MFMA_PEAK_TFLOPS = 10100.0  # MI355X dense fp4, published
FLUSH_BYTES = 512 * 2**20
COPY_BYTES = 2**30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {  # kernel -> sources whose text the measured counters belong to
    "paged_logits_kernel": ["paged_logits.hip", "device.h"],
    "paged_prefill_fp4_kernel": ["paged_prefill.hip", "device.h"],
    "mqa_logits_fp8_kernel": ["mqa_logits.hip", "device.h"],
}


def source_digest(kernel):
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "sparse_attention_indexer_mxfp4_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE passes,
    already scaled by the copy-kernel calibration; None when there is no entry or the
    kernel source has changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            table = json.load(f)
    except (OSError, ValueError):
        return None
    e = table.get(kernel, {}).get(workload)
    if not e or e.get("source_digest") != source_digest(kernel):
        return None
    return int(e["fetch_bytes"] + e["write_bytes"])


def copy_calibration():
    import torch
    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": COPY_BYTES, "copy_bytes_written": COPY_BYTES}), flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5, 6],
                   help="1-5: the indexer's five workloads; 6: the MXFP4 prefill chunk read off the paged cache")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--two-level", action="store_true",
                   help="time the two-level indexer on a paged workload instead: the source walk with block "
                        "maxima, the candidate pool, and a consumer that scores only the pool (prints its own "
                        "JSON line)")
    p.add_argument("--pool-blocks", type=int, default=64, help="two-level: candidate blocks per row")
    p.add_argument("--pool-block", type=int, default=64, help="two-level: keys per candidate block (16, 32, 64)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a plain 1 GiB device copy (the reference kernel for scaling "
                        "rocprofv3 FETCH_SIZE / WRITE_SIZE readings) and exit")
    return p.parse_args()


# ------------------------------------------------------------------------------------
# algorithmic work per launch
# ------------------------------------------------------------------------------------
def paged_work(wl, ends):
    """(keys scored, bytes, flop) of one paged logits launch: K read once per sequence,
    queries, weights, block-table entries, lengths, and the full-width logits written."""
    D, H = wl.D, wl.H
    per_key = D + 4 if wl.fmt == "fp8" else D // 2 + D // 32
    per_q = D if wl.fmt == "fp8" else D // 2 + 4 * (D // 32) // 4  # MXFP4: packed bytes + one int32 of scales
    seq_len = ends.reshape(wl.B, wl.next_n).max(axis=1)
    kbytes = int(seq_len.sum()) * per_key
    qbytes = wl.rows * H * per_q
    wbytes = wl.rows * H * 4
    btbytes = int(np.ceil(seq_len / wl.page_size).sum()) * 4
    lbytes = wl.B * 4
    obytes = wl.rows * wl.width * 4
    keys = int(ends.sum())
    flop = 2 * H * D * keys
    return keys, kbytes + qbytes + wbytes + btbytes + lbytes + obytes, flop


def prefill_paged_work(wl):
    """(keys scored, bytes, flop) of one paged prefill launch: the sequence's keys once,
    queries, weights, block-table entries, row ends, and the full logits written."""
    D, H, M = wl.D, wl.H, wl.M
    per_key = D + 4 if wl.fmt == "fp8" else D // 2 + D // 32
    per_q = D if wl.fmt == "fp8" else D // 2 + 4
    ends = np.clip(wl.row_end.astype(np.int64), 0, min(wl.width, wl.max_blocks * wl.page_size))
    n = int(ends.max(initial=0))
    keys = int(ends.sum())
    nbytes = n * per_key + M * H * (per_q + 4) + 4 * (-(-n // wl.page_size)) + 4 * M + 4 * M * wl.width
    return keys, nbytes, 2 * H * D * keys


def contig_work(wl):
    M, H, D, N = wl.M, wl.H, wl.D, wl.N
    keys = int(np.clip(wl.ke - wl.ks, 0, None).sum())
    nbytes = M * H * D + N * (D + 4) + 4 * M * H + 8 * M + 4 * M * N
    return keys, nbytes, 2 * H * D * keys


# ------------------------------------------------------------------------------------
# CPU oracle baseline (bounded sample)
# ------------------------------------------------------------------------------------
def cpu_baseline(cfg, wl, budget_s: float = 10.0):
    """The CPU oracle (float64 NumPy, BLAS per head) on a bounded sample of the same
    workload: whole sequences (paged) or blocks of query rows (contiguous), taken in
    order until about ``budget_s`` seconds of logits + top-k work have run.
    Quantisation of the sample's inputs is not timed."""
    from oracle import cache, formats, indexer

    threads = os.cpu_count()
    try:
        import threadpoolctl

        blas = [i["num_threads"] for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            threads = max(blas)
    except Exception:
        pass
    spent, keys, units, passes = 0.0, 0, 0, 0
    if cfg in (1, 4):
        kc, ks = formats.quantize_k_fp8(wl.k)
        step = 256 if cfg == 4 else wl.M
        qcache = {}
        while spent < budget_s:
            for r0 in range(0, wl.M, step):
                rows = np.arange(r0, min(wl.M, r0 + step))
                if r0 not in qcache:
                    qcache[r0] = formats.quantize_fp8_noscale(wl.q[rows])
                t0 = time.perf_counter()
                L = indexer.mqa_logits_fp8(qcache[r0], kc, ks, wl.w[rows], wl.ks[rows], wl.ke[rows])
                indexer.topk(L, wl.ks[rows], wl.ke[rows], wl.topk)
                spent += time.perf_counter() - t0
                keys += int(np.clip(wl.ke[rows] - wl.ks[rows], 0, None).sum())
                units = max(units, int(rows[-1]) + 1)
                if spent >= budget_s:
                    break
            else:
                passes += 1
        sample = (f"{passes} whole pass{'es' if passes > 1 else ''} over all {wl.M} query rows" if passes else f"query rows 0..{units - 1} of {wl.M}")
        sample += f" against all {wl.N} keys, logits + top-{wl.topk}"
    elif cfg == 6:
        P, D = wl.page_size, wl.D
        pool = np.zeros((wl.num_pages, cache.mxfp4_page_bytes(P, D)), np.uint8)
        packed, sb = formats.quantize_mxfp4(wl.k)
        cache.store_mxfp4(pool, wl.slot_mapping, packed, sb, P)
        step = 256
        for r0 in range(0, wl.M, step):
            rows = np.arange(r0, min(wl.M, r0 + step))
            q, qsb = formats.quantize_mxfp4(wl.q[rows])
            qs = formats.scales_to_int32(qsb)
            t0 = time.perf_counter()
            L = indexer.paged_logits(pool, wl.fmt, P, wl.block_table, wl.row_end[rows], q[None], wl.w[rows], 1,
                                     len(rows), wl.width, q_scale=qs[None], per_row=True)
            indexer.topk(L, None, wl.row_end[rows], wl.topk)
            spent += time.perf_counter() - t0
            keys += int(wl.row_end[rows].sum())
            units += len(rows)
            if spent >= budget_s:
                break
        sample = f"query rows 0..{units - 1} of {wl.M} against their paged keys, logits + top-{wl.topk}"
    else:
        # one pool for the sample: each sequence's keys are quantised into their own
        # pages the first time the sequence is visited (not timed); passes repeat over
        # the workload until the budget is spent
        P, D = wl.page_size, wl.D
        pb = cache.fp8_page_bytes(P, D) if wl.fmt == "fp8" else cache.mxfp4_page_bytes(P, D)
        pool = np.zeros((wl.num_pages, pb), np.uint8)
        prepared = {}
        while spent < budget_s:
            for b in range(wl.B):
                rows = np.arange(b * wl.next_n, (b + 1) * wl.next_n)
                if b not in prepared:
                    kr = np.arange(wl.key_offsets[b], wl.key_offsets[b] + wl.context_lens[b])
                    if wl.fmt == "fp8":
                        codes, sc = formats.quantize_k_fp8(wl.k[kr])
                        cache.store_fp8(pool, wl.slot_mapping[kr], codes, sc, P)
                        prepared[b] = (formats.quantize_fp8_noscale(wl.q[b:b + 1]), None)
                    else:
                        packed, sb = formats.quantize_mxfp4(wl.k[kr])
                        cache.store_mxfp4(pool, wl.slot_mapping[kr], packed, sb, P)
                        q, qsb = formats.quantize_mxfp4(wl.q[b:b + 1])
                        prepared[b] = (q, formats.scales_to_int32(qsb))
                q, qs = prepared[b]
                t0 = time.perf_counter()
                L = indexer.paged_logits(pool, wl.fmt, P, wl.block_table[b:b + 1], wl.context_lens[b:b + 1], q,
                                         wl.w[rows], 1, wl.next_n, wl.width, q_scale=qs)
                ends = indexer.paged_row_ends(wl.context_lens[b:b + 1], 1, wl.next_n)
                indexer.topk(L, None, ends, wl.topk)
                spent += time.perf_counter() - t0
                keys += int(ends.sum())
                units = max(units, b + 1)
                if spent >= budget_s:
                    break
            else:
                passes += 1
        sample = (f"{passes} whole pass{'es' if passes > 1 else ''} over all {wl.B} sequences" if passes else f"sequences 0..{units - 1} of {wl.B}")
        sample += f" ({keys} row-keys in all), logits + top-{wl.topk}"
    return {"value": round(keys / spent, 1), "unit": "keys/s", "cores": int(threads), "kind": "oracle",
            "sample": sample, "seconds": round(spent, 2)}


# ------------------------------------------------------------------------------------
# GPU
# ------------------------------------------------------------------------------------
def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the indexer path here has no multi-GPU mode (each GPU would "
              "score its own sequences independently); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return

    import torch

    from sparse_attention_indexer_mxfp4_amd import ops, workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = args.config
    wl = workloads.CONFIGS[cfg]() if cfg in workloads.CONFIGS else workloads.EXTRA[cfg]()
    paged = cfg in (2, 3, 5)
    if cfg == 6:
        return prefill_paged_main(args, wl, ops, torch, dev)

    if paged:
        fmt = ops.FP8 if wl.fmt == "fp8" else ops.MXFP4
        pb = ops.page_bytes(fmt, wl.page_size)
        copies = max(1, int(np.ceil(FLUSH_BYTES / (wl.num_pages * pb))))
        k_dev = torch.from_numpy(wl.k).to(dev)
        slots = torch.from_numpy(wl.slot_mapping).to(dev)
        pools = []
        for _ in range(copies):
            pool = torch.zeros((wl.num_pages, pb), dtype=torch.uint8, device=dev)
            ops.idx_k_store(pool, fmt, wl.page_size, k_dev, slots)  # quantise K with the library's own store
            pools.append(pool)
        # K store throughput (boundary op, timed on its own)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        ops.idx_k_store(pools[0], fmt, wl.page_size, k_dev, slots)
        e1.record()
        torch.cuda.synchronize()
        kstore_ms = e0.elapsed_time(e1)
        del k_dev
        q, q_scale = ops.idx_q_quant(torch.from_numpy(wl.q.reshape(-1, wl.H, wl.D)).to(dev), fmt)
        q = q.view(wl.B, wl.next_n, wl.H, -1).contiguous()
        if q_scale is not None:
            q_scale = q_scale.view(wl.B, wl.next_n, wl.H).contiguous()
        w = torch.from_numpy(wl.w).to(dev)
        ctx = torch.from_numpy(wl.context_lens).to(dev)
        bt = torch.from_numpy(wl.block_table).to(dev)
        rows = wl.rows
        logits = torch.empty((rows, (wl.width + 3) // 4 * 4), dtype=torch.float32, device=dev)[:, :wl.width]
        ends = torch.empty(rows, dtype=torch.int32, device=dev)
        out = torch.empty((rows, wl.topk), dtype=torch.int32, device=dev)

        def logits_call(i):
            ops.idx_paged_mqa_logits(pools[i % copies], fmt, wl.page_size, q, q_scale, w, ctx, bt, wl.width,
                                     logits=logits, row_end_out=ends)

        def topk_call():
            ops.idx_topk(logits, None, ends, wl.topk, out=out)

        if args.two_level:
            two_level(args, wl, ops, pools, copies, fmt, q, q_scale, w, ctx, bt, logits, ends, out, logits_call,
                      topk_call)
            return
        ends_host = None
    else:
        fmt = ops.FP8
        kq = torch.from_numpy(wl.k).to(dev)
        copies = max(1, int(np.ceil(FLUSH_BYTES / (wl.N * (wl.D + 4)))))
        qc, _ = ops.idx_q_quant(torch.from_numpy(wl.q).to(dev), fmt)
        # contiguous K: quantise through a page-size-16 pool and view its bytes back as rows
        P = 16
        npages = (wl.N + P - 1) // P
        kpools = []
        for _ in range(copies):
            pool = torch.zeros((npages, P * (wl.D + 4)), dtype=torch.uint8, device=dev)
            ops.idx_k_store(pool, fmt, P, kq, torch.arange(wl.N, dtype=torch.int64, device=dev))
            vals = pool[:, : P * wl.D].reshape(npages * P, wl.D)[: wl.N]
            scal = pool[:, P * wl.D:].contiguous().view(torch.float32).reshape(-1)[: wl.N]
            kpools.append((vals, scal.contiguous()))
        kstore_ms = None
        w = torch.from_numpy(wl.w).to(dev)
        ks = torch.from_numpy(wl.ks).to(dev)
        ke = torch.from_numpy(wl.ke).to(dev)
        logits = torch.empty((wl.M, (wl.N + 3) // 4 * 4), dtype=torch.float32, device=dev)[:, :wl.N]
        out = torch.empty((wl.M, wl.topk), dtype=torch.int32, device=dev)

        def logits_call(i):
            vals, scal = kpools[i % copies]
            ops.idx_mqa_logits(qc, vals, scal, w, ks, ke, logits=logits)

        def topk_call():
            ops.idx_topk(logits, ks, ke, wl.topk, out=out)

    # warmup
    for i in range(args.warmup):
        logits_call(i)
        topk_call()
    torch.cuda.synchronize()
    if paged:
        ends_host = ends.cpu().numpy()
        keys, nbytes, flop = paged_work(wl, ends_host)
    else:
        keys, nbytes, flop = contig_work(wl)

    stream = torch.cuda.current_stream()

    # (1) per-kernel durations with HIP events on the launch stream: the K launches of
    # each kernel captured back to back in a HIP graph of their own, one untimed
    # replay, then one replay between two events (an event pair per launch would cost
    # as much as a decode launch, and launches enqueued from Python could leave the
    # GPU idle between kernels)
    def timed_replay(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(args.steps):
                fn(i)
        g.replay()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        g.replay()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / args.steps

    logits_ms = timed_replay(logits_call)
    topk_ms = timed_replay(lambda i: topk_call())

    # (2) whole-step throughput: the K timed steps captured in one HIP graph (the
    # calls neither allocate nor synchronise) and replayed once, so the host's
    # per-launch cost does not pace the GPU
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(args.steps):
            logits_call(i)
            topk_call()
    graph.replay()  # untimed first replay
    torch.cuda.synchronize()
    step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    t0 = time.perf_counter()
    step_ev[0].record(stream)
    graph.replay()
    step_ev[1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    b2b_ms = logits_ms
    logits_ms = in_step(step_ev[0].elapsed_time(step_ev[1]) / args.steps, topk_ms, b2b_ms)

    ms_per_step = elapsed * 1e3 / args.steps
    value = keys * args.steps / elapsed
    if cfg == 4 or cfg == 1:
        achieved = flop / (logits_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": FP8_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / FP8_MFMA_PEAK_TFLOPS, 4),
                "traffic": measured_traffic("mqa_logits_fp8_kernel", wl.name),
                "kernel": "mqa_logits_fp8_kernel", "kernel_ms": round(logits_ms, 4),
                "algorithmic_flop": flop, "algorithmic_bytes": nbytes}
    else:
        achieved = nbytes / (logits_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic("paged_logits_kernel", wl.name), "kernel": "paged_logits_kernel",
                "kernel_ms": round(logits_ms, 4), "algorithmic_bytes": nbytes, "algorithmic_flop": flop}
    result = {
        "metric": "indexer keys scored/sec + decode HBM GB/s (% of peak), 1 MI355X",
        "value": round(value, 1),
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if wl_fmt(wl, cfg) == "fp8" else "fp4",
        "data": "synthetic",
        "config": {"workload": wl.name, "config": cfg, "keys_per_step": keys, "topk": wl.topk,
                   "timing": TIMING, "logits_ms": round(logits_ms, 4), "logits_b2b_ms": round(b2b_ms, 4),
                   "topk_ms": round(topk_ms, 4),
                   "kstore_ms": None if kstore_ms is None else round(kstore_ms, 4), "k_cache_copies": copies},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, wl)
    print(json.dumps(result), flush=True)


def prefill_paged_main(args, wl, ops, torch, dev):
    """The prefill chunk read straight off the paged MXFP4 cache: logits + top-k per step."""
    fmt = ops.MXFP4
    pb = ops.page_bytes(fmt, wl.page_size)
    copies = max(1, int(np.ceil(FLUSH_BYTES / (wl.num_pages * pb))))
    k_dev = torch.from_numpy(wl.k).to(dev)
    slots = torch.from_numpy(wl.slot_mapping).to(dev)
    pools = []
    for _ in range(copies):
        pool = torch.zeros((wl.num_pages, pb), dtype=torch.uint8, device=dev)
        ops.idx_k_store(pool, fmt, wl.page_size, k_dev, slots)
        pools.append(pool)
    del k_dev
    q, q_scale = ops.idx_q_quant(torch.from_numpy(wl.q).to(dev), fmt)
    w = torch.from_numpy(wl.w).to(dev)
    ends = torch.from_numpy(wl.row_end).to(dev)
    bt = torch.from_numpy(wl.block_table[0]).to(dev)
    logits = torch.empty((wl.M, (wl.width + 3) // 4 * 4), dtype=torch.float32, device=dev)[:, :wl.width]
    out = torch.empty((wl.M, wl.topk), dtype=torch.int32, device=dev)

    def logits_call(i):
        ops.idx_paged_prefill_logits(pools[i % copies], fmt, wl.page_size, q, q_scale, w, ends, bt, wl.width,
                                     logits=logits)

    def topk_call(i):
        ops.idx_topk(logits, None, ends, wl.topk, out=out)

    for i in range(args.warmup):
        logits_call(i)
        topk_call(i)
    torch.cuda.synchronize()
    keys, nbytes, flop = prefill_paged_work(wl)
    logits_ms = timed_graph(torch, logits_call, args.steps)
    topk_ms = timed_graph(torch, topk_call, args.steps)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(args.steps):
            logits_call(i)
            topk_call(i)
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    t0 = time.perf_counter()
    step_ev[0].record(stream)
    g.replay()
    step_ev[1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    b2b_ms = logits_ms
    logits_ms = in_step(step_ev[0].elapsed_time(step_ev[1]) / args.steps, topk_ms, b2b_ms)
    achieved = flop / (logits_ms * 1e-3) / 1e12
    result = {
        "metric": "indexer keys scored/sec, prefill chunk off the paged MXFP4 cache, 1 MI355X",
        "value": round(keys * args.steps / elapsed, 1),
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4",
        "data": "synthetic",
        "config": {"workload": wl.name, "config": 6, "keys_per_step": keys, "topk": wl.topk,
                   "timing": TIMING, "logits_ms": round(logits_ms, 4), "logits_b2b_ms": round(b2b_ms, 4),
                   "topk_ms": round(topk_ms, 4), "k_cache_copies": copies},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": FP4_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / FP4_MFMA_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic("paged_prefill_fp4_kernel", wl.name),
                     "kernel": "paged_prefill_fp4_kernel", "kernel_ms": round(logits_ms, 4),
                     "algorithmic_flop": flop, "algorithmic_bytes": nbytes},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(6, wl, budget_s=5.0)
    print(json.dumps(result), flush=True)


TIMING = ("K steps in one HIP graph, timed with HIP events on the launch stream; top-k time from HIP events "
          "around a graph of K back-to-back top-k launches; logits time inside the step = step time - top-k time "
          "(logits_b2b_ms: a graph of K back-to-back logits launches)")


def in_step(step_ms, topk_ms, b2b_ms):
    """Logits time per launch inside the timed step: the step's HIP-event time less the
    top-k's back-to-back time (the back-to-back logits figure if that leaves nothing)."""
    d = step_ms - topk_ms
    return d if d > 0 else b2b_ms


def timed_graph(torch, fn, steps):
    """Per-launch duration (ms) of fn(i), i < steps, captured back to back in one HIP graph:
    one untimed replay, then one replay between two HIP events on the launch stream."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    g.replay()
    ev[1].record(stream)
    torch.cuda.synchronize()
    return ev[0].elapsed_time(ev[1]) / steps


def two_level(args, wl, ops, pools, copies, fmt, q, q_scale, w, ctx, bt, logits, ends, out, logits_call, topk_call):
    """The two-level indexer on one paged step: a source layer (the dense walk that also
    writes block maxima, then the pool: each row's best blocks) and one consumer layer
    that scores only the pool (gathered walk, top-k over the pool, remap to positions),
    next to the same consumer run densely (logits + top-k over the whole context)."""
    import torch

    dev = q.device
    block, n = args.pool_block, args.pool_blocks
    rows = wl.rows
    nb = -(-wl.width // block)
    bm = torch.empty((rows, nb), dtype=torch.float32, device=dev)
    cand = torch.empty((rows, n), dtype=torch.int32, device=dev)
    pw = n * block
    pool = torch.empty((rows, pw), dtype=torch.float32, device=dev)
    pend = torch.empty(rows, dtype=torch.int32, device=dev)
    pout = torch.empty((rows, wl.topk), dtype=torch.int32, device=dev)

    def source(i):
        ops.idx_paged_mqa_logits_block_max(pools[i % copies], fmt, wl.page_size, q, q_scale, w, ctx, bt, wl.width,
                                           block, logits=logits, row_end_out=ends, block_max=bm)

    def select(i):
        ops.idx_candidate_blocks(bm, ends, block, n, out=cand)

    def gather(i):
        ops.idx_paged_mqa_logits_gather(pools[i % copies], fmt, wl.page_size, q, q_scale, w, ctx, bt, cand, block,
                                        pool_logits=pool, pool_end=pend)

    def pool_topk(i):
        ops.idx_topk(pool, None, pend, wl.topk, out=pout)

    def remap(i):
        ops.idx_remap_compact_topk(pout, cand, block)

    for i in range(args.warmup):
        source(i); select(i); gather(i); pool_topk(i); remap(i)
    torch.cuda.synchronize()
    # algorithmic bytes of the gathered walk: each row reads the keys its pool names
    # (once per row), its queries and weights, one candidate entry per block and one
    # block-table entry per 16-key group; it writes the whole pool row
    e = ends.cpu().numpy().astype(np.int64)
    c = cand.cpu().numpy().astype(np.int64)
    nbe = -(-e // block)
    ok = (c >= 0) & (c < nbe[:, None])
    keys_per_row = np.where(ok, np.minimum(block, e[:, None] - c * block), 0).sum(axis=1)
    pool_keys = int(keys_per_row.sum())
    D, H = wl.D, wl.H
    per_key = D + 4 if wl.fmt == "fp8" else D // 2 + D // 32
    per_q = D if wl.fmt == "fp8" else D // 2 + 4
    gbytes = (pool_keys * per_key + rows * H * (per_q + 4) + rows * n * 4 + int(np.ceil(keys_per_row / 16).sum()) * 4
              + rows * 8 + rows * pw * 4)
    dense_keys, _, _ = paged_work(wl, e)

    t = {name: timed_graph(torch, fn, args.steps) for name, fn in
         (("dense_logits", logits_call), ("dense_topk", lambda i: topk_call()), ("source", source),
          ("select", select), ("gather", gather), ("pool_topk", pool_topk), ("remap", remap))}

    def consumer(i):
        gather(i); pool_topk(i); remap(i)

    consumer_ms = timed_graph(torch, consumer, args.steps)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(args.steps):
            source(i); select(i); consumer(i)
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    step_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    achieved = gbytes / (t["gather"] * 1e-3) / 1e9
    result = {
        "metric": "two-level indexer consumer: pool keys scored/sec (gathered walk + top-k + remap), 1 MI355X",
        "value": round(pool_keys / (consumer_ms * 1e-3), 1),
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if wl.fmt == "fp8" else "fp4",
        "data": "synthetic",
        "config": {"workload": wl.name + f" two-level pool {n}x{block}", "pool_blocks": n, "pool_block": block,
                   "topk": wl.topk, "pool_keys_per_step": pool_keys, "dense_keys_per_step": dense_keys,
                   "timing": "step = source + pool + consumer, K steps in one HIP graph; per-kernel times from HIP "
                             "events around a graph of K back-to-back launches of that call",
                   "source_ms": round(t["source"], 4), "dense_logits_ms": round(t["dense_logits"], 4),
                   "select_ms": round(t["select"], 4), "gather_ms": round(t["gather"], 4),
                   "pool_topk_ms": round(t["pool_topk"], 4), "remap_ms": round(t["remap"], 4),
                   "consumer_ms": round(consumer_ms, 4),
                   "dense_consumer_ms": round(t["dense_logits"] + t["dense_topk"], 4), "k_cache_copies": copies},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("paged_logits_kernel", wl.name + f" two-level pool {n}x{block}"),
                     "kernel": "paged_logits_kernel (gathered walk)", "kernel_ms": round(t["gather"], 4),
                     "algorithmic_bytes": gbytes},
    }
    print(json.dumps(result), flush=True)


def wl_fmt(wl, cfg):
    return getattr(wl, "fmt", "fp8")


if __name__ == "__main__":
    main()
