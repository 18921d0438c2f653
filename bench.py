"""Indexer benchmark on one MI355X: keys scored per second for one whole indexer step
(logits over every cached key, causal masks, per-row top-k) on seeded synthetic
workloads, with the dominant kernel's roofline fraction and the CPU oracle beside it.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config N] [--headline-only]
                    [--no-cpu-baseline] [--no-calibration]

Default: the headline is the paged fp8 MTP decode step (128 sequences x 2 rows,
context lengths log-uniform on [4096, 65536], 64 heads, logits width 65536,
top-2048), the largest decode workload; the line also carries the fp8 decode
(B = 32), the fp8 prefill chunk (8192 x 8192), the MXFP4 decode (B = 64) and the
MXFP4 prefill chunk read off the paged cache (8192 x 8192) as sub-objects under
"configs", each with its own roofline and CPU oracle baseline, and
the ceilings measured on this GPU (streaming copy / read, fp8 / fp4 matrix loops)
under "calibration". ``--config N`` prints one workload's line instead (1-5: the five
workloads; 6: the MXFP4 prefill chunk read off the paged cache). Inputs live in HBM
before timing starts. Each timed step reads a different copy of the K cache (copies
totalling more than 512 MB rotate), so the 256 MB Infinity Cache cannot hold a step's
keys from the previous visit.

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
    p.add_argument("--config", type=int, default=None, choices=[1, 2, 3, 4, 5, 6],
                   help="one workload's line only (1-5: the indexer's five workloads; 6: the MXFP4 prefill chunk "
                        "read off the paged cache); default: the MTP headline with the others as sub-objects")
    p.add_argument("--headline-only", action="store_true", help="default mode without the sub-objects")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-calibration", action="store_true", help="skip the measured copy / matrix-core ceilings")
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
# measured ceilings of this device
# ------------------------------------------------------------------------------------
def calibration(torch):
    """HBM and matrix-core ceilings measured on this GPU with libidx_calib's kernels
    (include/idx_calib.h): a streaming copy and a streaming read of 2 GiB (above the
    256 MB Infinity Cache), and the dense 16x16x128 fp8 and fp4 matrix loops, each the
    median of 5 launches timed with HIP events on the launch stream."""
    import ctypes

    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_attention_indexer_mxfp4_amd", "libidx_calib.so"))
    P, SZ, I32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    lib.idx_calib_copy.argtypes = [P, P, SZ, P]
    lib.idx_calib_read.argtypes = [P, SZ, P, P]
    lib.idx_calib_mfma.argtypes = [I32, I32, P, ctypes.POINTER(ctypes.c_int64), P]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream
    nbytes = 2 * 2**30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    sink = torch.empty(8192, dtype=torch.float32, device=dev)

    def timed(fn, reps=5):
        rc = fn()
        if rc != 0:
            raise RuntimeError(f"calibration kernel failed: {rc}")
        ts = []
        for _ in range(reps):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(stream)
            fn()
            ev[1].record(stream)
            torch.cuda.synchronize()
            ts.append(ev[0].elapsed_time(ev[1]))
        return sorted(ts)[len(ts) // 2] * 1e-3

    t_copy = timed(lambda: lib.idx_calib_copy(src.data_ptr(), dst.data_ptr(), nbytes, s))
    t_read = timed(lambda: lib.idx_calib_read(src.data_ptr(), nbytes, sink.data_ptr(), s))
    del src, dst
    out = {"copy_GBps": round(2 * nbytes / t_copy / 1e9, 1), "read_GBps": round(nbytes / t_read / 1e9, 1),
           "hbm_spec_GBps": HBM_PEAK_GBS}
    for fmt, name, spec in ((0, "fp8", FP8_MFMA_PEAK_TFLOPS), (1, "fp4", FP4_MFMA_PEAK_TFLOPS)):
        flop = ctypes.c_int64(0)
        t = timed(lambda: lib.idx_calib_mfma(fmt, 4000, sink.data_ptr(), ctypes.byref(flop), s))
        out[f"{name}_mfma_TFLOPs"] = round(flop.value / t / 1e12, 1)
        out[f"{name}_mfma_spec_TFLOPs"] = spec
    out["method"] = ("libidx_calib: 2 GiB streaming copy (bytes read + written) and read, 16-byte loads, 8 "
                     "workgroups per CU; dense 16x16x128 fp8 / fp4 matrix loops from register operands, 8 waves "
                     "per CU; median of 5 launches, HIP events")
    return out


# ------------------------------------------------------------------------------------
# GPU
# ------------------------------------------------------------------------------------
SUB_CONFIGS = (2, 4, 5, 6)


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
    cfg = 3 if args.config is None else args.config
    if args.two_level:
        wl = workloads.CONFIGS[cfg]()
        st = setup_paged(wl, ops, torch, dev)
        two_level(args, wl, ops, st["pools"], st["copies"], st["fmt"], st["q"], st["q_scale"], st["w"], st["ctx"],
                  st["bt"], st["logits"], st["ends"], st["out"], st["logits_call"], st["topk_call"])
        return

    head = measure(cfg, args, ops, workloads, torch, dev, cpu_budget=10.0, one_thread_budget=4.0)
    result = {
        "metric": "indexer keys scored/sec + decode HBM GB/s (% of peak), 1 MI355X",
        "value": head["value"],
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": head["config"],
        "roofline": head["roofline"],
    }
    if "cpu_baseline" in head:
        result["cpu_baseline"] = head["cpu_baseline"]
    if args.config is None and not args.headline_only:
        subs = {}
        for c in SUB_CONFIGS:
            torch.cuda.empty_cache()
            subs[str(c)] = measure(c, args, ops, workloads, torch, dev, cpu_budget=5.0, one_thread_budget=0.0)
        result["configs"] = subs
    if not args.no_calibration:
        torch.cuda.empty_cache()
        cal = calibration(torch)
        result["calibration"] = cal
        for part in [result] + list(result.get("configs", {}).values()):
            roof = part["roofline"]
            if roof["bound"] == "hbm":
                roof["measured_ceiling"] = cal["read_GBps"]
            else:
                roof["measured_ceiling"] = cal["fp8_mfma_TFLOPs" if roof["peak"] == FP8_MFMA_PEAK_TFLOPS
                                              else "fp4_mfma_TFLOPs"]
            roof["frac_of_measured_ceiling"] = round(roof["achieved"] / roof["measured_ceiling"], 4)
    print(json.dumps(result), flush=True)


def setup_paged(wl, ops, torch, dev):
    """Device inputs of a paged step: K-cache copies quantised by the library's own K
    store (copies totalling more than FLUSH_BYTES rotate), queries, weights, lengths,
    block table, and the logits / row-end / top-k outputs, with the two calls."""
    fmt = ops.FP8 if wl.fmt == "fp8" else ops.MXFP4
    pb = ops.page_bytes(fmt, wl.page_size)
    copies = max(1, int(np.ceil(FLUSH_BYTES / (wl.num_pages * pb))))
    k_dev = torch.from_numpy(wl.k).to(dev)
    slots = torch.from_numpy(wl.slot_mapping).to(dev)
    pools = []
    for _ in range(copies):
        pool = torch.zeros((wl.num_pages, pb), dtype=torch.uint8, device=dev)
        ops.idx_k_store(pool, fmt, wl.page_size, k_dev, slots)
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

    def topk_call(i):
        ops.idx_topk(logits, None, ends, wl.topk, out=out)

    return dict(fmt=fmt, pools=pools, copies=copies, q=q, q_scale=q_scale, w=w, ctx=ctx, bt=bt, logits=logits,
                ends=ends, out=out, logits_call=logits_call, topk_call=topk_call, kstore_ms=kstore_ms)


def setup_contig(wl, ops, torch, dev):
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
    w = torch.from_numpy(wl.w).to(dev)
    ks = torch.from_numpy(wl.ks).to(dev)
    ke = torch.from_numpy(wl.ke).to(dev)
    logits = torch.empty((wl.M, (wl.N + 3) // 4 * 4), dtype=torch.float32, device=dev)[:, :wl.N]
    out = torch.empty((wl.M, wl.topk), dtype=torch.int32, device=dev)

    def logits_call(i):
        vals, scal = kpools[i % copies]
        ops.idx_mqa_logits(qc, vals, scal, w, ks, ke, logits=logits)

    def topk_call(i):
        ops.idx_topk(logits, ks, ke, wl.topk, out=out)

    return dict(copies=copies, logits_call=logits_call, topk_call=topk_call, kstore_ms=None)


def setup_prefill_paged(wl, ops, torch, dev):
    """The prefill chunk read straight off the paged cache (config 6: MXFP4)."""
    fmt = ops.FP8 if wl.fmt == "fp8" else ops.MXFP4
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

    return dict(copies=copies, logits_call=logits_call, topk_call=topk_call, kstore_ms=None, ends=ends)


def measure(cfg, args, ops, workloads, torch, dev, cpu_budget, one_thread_budget):
    """One workload: K steps (logits + top-k) in one HIP graph timed with HIP events on
    the launch stream, the two kernels' back-to-back times, the dominant kernel's
    roofline and the CPU oracle on a bounded sample. Returns the workload's part of
    the JSON line."""
    wl = workloads.CONFIGS[cfg]() if cfg in workloads.CONFIGS else workloads.EXTRA[cfg]()
    paged = cfg in (2, 3, 5)
    if paged:
        st = setup_paged(wl, ops, torch, dev)
    elif cfg == 6:
        st = setup_prefill_paged(wl, ops, torch, dev)
    else:
        st = setup_contig(wl, ops, torch, dev)
    logits_call, topk_call = st["logits_call"], st["topk_call"]

    for i in range(args.warmup):
        logits_call(i)
        topk_call(i)
    torch.cuda.synchronize()
    if paged:
        keys, nbytes, flop = paged_work(wl, st["ends"].cpu().numpy())
    elif cfg == 6:
        keys, nbytes, flop = prefill_paged_work(wl)
    else:
        keys, nbytes, flop = contig_work(wl)

    # per-kernel durations: K launches of one kernel back to back in a HIP graph of
    # their own, one untimed replay, then one replay between two HIP events
    b2b_ms = timed_graph(torch, logits_call, args.steps)
    topk_ms = timed_graph(torch, topk_call, args.steps)

    # whole-step throughput: the K timed steps captured in one HIP graph (the calls
    # neither allocate nor synchronise) and replayed once, so the host's per-launch
    # cost does not pace the GPU
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(args.steps):
            logits_call(i)
            topk_call(i)
    graph.replay()  # untimed first replay
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    t0 = time.perf_counter()
    step_ev[0].record(stream)
    graph.replay()
    step_ev[1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = step_ev[0].elapsed_time(step_ev[1]) / args.steps
    logits_ms = in_step(step_ms, topk_ms, b2b_ms)
    del graph

    fmt = wl_fmt(wl, cfg)
    if cfg in (1, 4, 6):
        kernel = "mqa_logits_fp8_kernel" if cfg != 6 else "paged_prefill_fp4_kernel"
        peak = FP8_MFMA_PEAK_TFLOPS if fmt == "fp8" else FP4_MFMA_PEAK_TFLOPS
        achieved = flop / (logits_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": measured_traffic(kernel, wl.name),
                "kernel": kernel, "kernel_ms": round(logits_ms, 4),
                "frac_b2b": round(flop / (b2b_ms * 1e-3) / 1e12 / peak, 4), "kernel_ms_b2b": round(b2b_ms, 4),
                "algorithmic_flop": flop, "algorithmic_bytes": nbytes}
    else:
        achieved = nbytes / (logits_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic("paged_logits_kernel", wl.name), "kernel": "paged_logits_kernel",
                "kernel_ms": round(logits_ms, 4),
                "frac_b2b": round(nbytes / (b2b_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "kernel_ms_b2b": round(b2b_ms, 4), "algorithmic_bytes": nbytes, "algorithmic_flop": flop}
    part = {
        "value": round(keys * args.steps / elapsed, 1),
        "unit": "keys/s",
        "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
        "dtype": "fp8" if fmt == "fp8" else "fp4",
        "config": {"workload": wl.name, "config": cfg, "keys_per_step": keys, "topk": wl.topk, "timing": TIMING,
                   "step_ms": round(step_ms, 4), "logits_ms": round(logits_ms, 4), "logits_b2b_ms": round(b2b_ms, 4),
                   "topk_ms": round(topk_ms, 4),
                   "kstore_ms": None if st["kstore_ms"] is None else round(st["kstore_ms"], 4),
                   "k_cache_copies": st["copies"]},
        "roofline": roof,
    }
    del st
    if not args.no_cpu_baseline:
        cb = cpu_baseline(cfg, wl, budget_s=cpu_budget)
        cb["cpu_model"] = cpu_model()
        if one_thread_budget > 0:
            try:
                import threadpoolctl

                with threadpoolctl.threadpool_limits(limits=1):
                    one = cpu_baseline(cfg, wl, budget_s=one_thread_budget)
                cb["one_thread"] = {"value": one["value"], "unit": "keys/s", "cores": 1, "sample": one["sample"],
                                    "seconds": one["seconds"]}
            except ImportError:
                pass
        part["cpu_baseline"] = cb
    return part


def cpu_model():
    """The host CPU's model name (what lscpu reports as "Model name")."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


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
         (("dense_logits", logits_call), ("dense_topk", topk_call), ("source", source),
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
