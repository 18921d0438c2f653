"""Quantised indexer inputs for the tests, prepared on the CPU by the oracle.

Raw draws come from the workload generator (no indexer arithmetic); every code,
scale and cache byte handed to the GPU here is produced by ``oracle`` code, so no
expected value depends on the HIP path.
"""

from __future__ import annotations

import concurrent.futures
from dataclasses import dataclass

import numpy as np

from oracle import cache, formats

CHUNK = 65536
_POOL = concurrent.futures.ThreadPoolExecutor(max_workers=8)


def _chunked(fn, x, *outs_shape):
    n = x.shape[0]
    parts = list(_POOL.map(lambda i: fn(x[i:i + CHUNK]), range(0, n, CHUNK)))
    if not parts:
        return fn(x)
    if isinstance(parts[0], tuple):
        return tuple(np.concatenate([p[j] for p in parts]) for j in range(len(parts[0])))
    return np.concatenate(parts)


def quant_k_fp8(k):
    return _chunked(formats.quantize_k_fp8, k)


def quant_mxfp4(x):
    flat = x.reshape(-1, x.shape[-1])
    packed, bits = _chunked(formats.quantize_mxfp4, flat)
    return packed.reshape(x.shape[:-1] + (x.shape[-1] // 2,)), bits.reshape(x.shape[:-1] + (x.shape[-1] // 32,))


def quant_q_fp8(q):
    flat = q.reshape(-1, q.shape[-1])
    return _chunked(formats.quantize_fp8_noscale, flat).reshape(q.shape)


@dataclass
class PagedInputs:
    wl: object
    pool: np.ndarray  # [num_pages, stride] uint8
    q: np.ndarray  # fp8 [B, next_n, H, D] or MXFP4 packed [B, next_n, H, D/2]
    q_scale: np.ndarray | None  # MXFP4 [B, next_n, H] int32
    k_codes: np.ndarray  # fp8 [Nk, D] or packed [Nk, D/2]
    k_scales: np.ndarray  # fp8 [Nk] f32 or MXFP4 [Nk, D/32] uint8


def paged_inputs(wl, stride_pad: int = 0) -> PagedInputs:
    P, D = wl.page_size, wl.D
    if wl.fmt == "fp8":
        pool = np.zeros((wl.num_pages, cache.fp8_page_bytes(P, D) + stride_pad), np.uint8)
        codes, sc = quant_k_fp8(wl.k)
        for i in range(0, codes.shape[0], CHUNK):
            cache.store_fp8(pool, wl.slot_mapping[i:i + CHUNK], codes[i:i + CHUNK], sc[i:i + CHUNK], P)
        return PagedInputs(wl, pool, quant_q_fp8(wl.q), None, codes, sc)
    pool = np.zeros((wl.num_pages, cache.mxfp4_page_bytes(P, D) + stride_pad), np.uint8)
    packed, sb = quant_mxfp4(wl.k)
    for i in range(0, packed.shape[0], CHUNK):
        cache.store_mxfp4(pool, wl.slot_mapping[i:i + CHUNK], packed[i:i + CHUNK], sb[i:i + CHUNK], P)
    qp, qsb = quant_mxfp4(wl.q)
    return PagedInputs(wl, pool, qp, formats.scales_to_int32(qsb), packed, sb)


@dataclass
class ContigInputs:
    wl: object
    q: np.ndarray  # [M, H, D] e4m3
    k: np.ndarray  # [N, D] e4m3
    k_scale: np.ndarray  # [N] f32


def contig_inputs(wl) -> ContigInputs:
    codes, sc = quant_k_fp8(wl.k)
    return ContigInputs(wl, quant_q_fp8(wl.q), codes, sc)
