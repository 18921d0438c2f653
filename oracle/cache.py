"""Byte layout of one paged indexer K cache entry, as a writer and a reader.

TEST INFRASTRUCTURE ONLY (see the package docstring).

A pool is a uint8 array [num_pages, page_stride]; ``page_stride`` may exceed the bytes
a page needs (the pool's stride, as ``_kv_view`` on page
``vllm.v1.attention.ops.rocm_paged_mxfp4_indexer`` notes). Key slot ``slot`` is entry
``slot % P`` of page ``slot // P``.

fp8 block-flat page (page ``vllm.v1.attention.ops.rocm_aiter_mla_sparse``,
``rocm_fp8_paged_mqa_logits`` and ``rocm_fp8_paged_mqa_logits_triton``: a
[blocks, P, 1, D + 4] uint8 page read as P*D e4m3 bytes followed by fp32 scales):
entry u's D value bytes start at u*D; its fp32 scale (little-endian) at P*D + 4u.

MXFP4 page (page ``vllm.v1.attention.ops.rocm_paged_mxfp4_indexer``,
``RocmPagedMxfp4CacheLayout`` and ``rocm_paged_mxfp4_cache_layout``): D/2 packed bytes
and D/32 e8m0 bytes per entry. The page is cut into runs of n_per_tile = 16 entries;
inside a run the packed bytes are stored [chunk, entry, byte] with 16-byte chunks, and
the scales [scale % scale_lanes, entry, scale // scale_lanes] with
scale_lanes = 64 // n_per_tile = 4 (the wavefront is 64 lanes on gfx950). The value
bytes of all runs come first and the scale bytes of all runs follow them, the way the
fp8 page puts its scales after its values; the pages give the orders inside a run but
not where the scale region sits, and this is the reading taken.
"""

from __future__ import annotations

import numpy as np

N_PER_TILE = 16
D_PER_TILE = 16
SCALE_LANES = 64 // N_PER_TILE


def fp8_page_bytes(P: int, D: int) -> int:
    return P * (D + 4)


def mxfp4_page_bytes(P: int, D: int) -> int:
    return P * (D // 2 + D // 32)


def _fp8_offsets(P: int, D: int, entry: np.ndarray):
    vals = entry[:, None] * D + np.arange(D)[None, :]
    scale = P * D + 4 * entry[:, None] + np.arange(4)[None, :]
    return vals, scale


def _mxfp4_offsets(P: int, D: int, entry: np.ndarray):
    if P % N_PER_TILE or (D // 2) % D_PER_TILE or (D // 32) % SCALE_LANES:
        raise ValueError("page geometry the MXFP4 run layout cannot express")
    nb = D // 2  # packed bytes per entry
    ns = D // 32  # scale bytes per entry
    run = entry // N_PER_TILE
    tok = entry % N_PER_TILE
    j = np.arange(nb)
    chunk, beta = j // D_PER_TILE, j % D_PER_TILE
    vals = (run[:, None] * (N_PER_TILE * nb) + chunk[None, :] * (N_PER_TILE * D_PER_TILE)
            + tok[:, None] * D_PER_TILE + beta[None, :])
    i = np.arange(ns)
    per_lane = ns // SCALE_LANES
    scale = (P * nb + run[:, None] * (N_PER_TILE * ns) + (i % SCALE_LANES)[None, :] * (N_PER_TILE * per_lane)
             + tok[:, None] * per_lane + (i // SCALE_LANES)[None, :])
    return vals, scale


def _split_slots(slots, P: int, num_pages: int):
    slots = np.asarray(slots, dtype=np.int64)
    page = slots // P
    entry = slots % P
    if np.any((page < 0) | (page >= num_pages)):
        raise ValueError("slot outside the pool")
    return page, entry


def store_fp8(pool: np.ndarray, slots, codes, scales, P: int) -> None:
    """Write e4m3 rows ``codes`` [N, D] and fp32 ``scales`` [N] at ``slots`` [N].
    Negative slots are skipped (padding)."""
    slots = np.asarray(slots, dtype=np.int64)
    keep = slots >= 0
    codes = np.asarray(codes, dtype=np.uint8)[keep]
    sc = np.asarray(scales, dtype=np.float32)[keep].view(np.uint8).reshape(-1, 4)
    page, entry = _split_slots(slots[keep], P, pool.shape[0])
    D = codes.shape[1]
    vo, so = _fp8_offsets(P, D, entry)
    pool[page[:, None], vo] = codes
    pool[page[:, None], so] = sc


def load_fp8(pool: np.ndarray, slots, P: int, D: int):
    """Read e4m3 rows [N, D] and fp32 scales [N] at ``slots``."""
    page, entry = _split_slots(slots, P, pool.shape[0])
    vo, so = _fp8_offsets(P, D, entry)
    codes = pool[page[:, None], vo]
    scales = np.ascontiguousarray(pool[page[:, None], so]).view(np.float32).reshape(-1)
    return codes, scales


def store_mxfp4(pool: np.ndarray, slots, packed, scale_bytes, P: int) -> None:
    """Write packed e2m1 rows [N, D/2] and e8m0 bytes [N, D/32] at ``slots``.
    Negative slots are skipped (padding)."""
    slots = np.asarray(slots, dtype=np.int64)
    keep = slots >= 0
    packed = np.asarray(packed, dtype=np.uint8)[keep]
    sb = np.asarray(scale_bytes, dtype=np.uint8)[keep]
    page, entry = _split_slots(slots[keep], P, pool.shape[0])
    D = packed.shape[1] * 2
    vo, so = _mxfp4_offsets(P, D, entry)
    pool[page[:, None], vo] = packed
    pool[page[:, None], so] = sb


def load_mxfp4(pool: np.ndarray, slots, P: int, D: int):
    """Read packed e2m1 rows [N, D/2] and e8m0 bytes [N, D/32] at ``slots``."""
    page, entry = _split_slots(slots, P, pool.shape[0])
    vo, so = _mxfp4_offsets(P, D, entry)
    return pool[page[:, None], vo], pool[page[:, None], so]
