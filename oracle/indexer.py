"""Indexer logits, row ranges and per-row top-k, by their definitions, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Logits (page ``vllm.v1.attention.ops.rocm_aiter_mla_sparse``, ``fp8_mqa_logits_torch``):
for each head the score of key s for row t is the dot product of the dequantised query
head and the dequantised key, times the key's per-token scale; the logit is the sum over
heads of the head weight times the ReLU of that score; columns outside the row's
[start, end) are -inf. The weights arrive with the softmax and head scales already
folded in (page ``vllm.v1.attention.ops.rocm_paged_mxfp4_indexer``,
``rocm_mxfp4_sparse_attn_indexer``), so nothing else multiplies the logit.

The per-head dot products are exact in float64 for these formats (e4m3 x e4m3 products
have at most 8 significant bits, MXFP4 ones fewer, and a 128-term sum of them spans far
fewer than 53 bits); only the head sum rounds. The method approximates nothing beyond
the quantisation of its inputs, so this module is the definition written out.

Unlike ``fp8_mqa_logits_torch``, which rounds each per-head score to bf16 on its way
through ``einsum``, nothing here rounds before the head sum.
"""

from __future__ import annotations

import numpy as np

from . import cache, formats


# ----------------------------------------------------------------------------------
# logits
# ----------------------------------------------------------------------------------
def logits_from_values(q, k, w, starts, ends, k_scale=None, width=None, magnitude: bool = False) -> np.ndarray:
    """I[t, s] = sum_h w[t, h] * max(k_scale[s] * (q[t, h, :] . k[s, :]), 0) on
    [starts[t], ends[t]), -inf elsewhere.

    q is [M, H, D] and k is [N, D], both already dequantised to float64; k_scale is
    [N] or None (1.0). The result is [M, width] (width defaults to N); columns at or
    beyond N are -inf. Row ranges are clipped to [0, min(N, width)).

    With ``magnitude`` the same walk returns instead
    A[t, s] = sum_h |w[t, h]| * k_scale[s] * sum_d |q[t, h, d] * k[s, d]|, the scale of
    the rounding error any summation-based evaluation of I[t, s] carries (the
    tolerance of the parity tests is stated against it for ill-conditioned rows).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    M, H, _ = q.shape
    N = k.shape[0]
    width = N if width is None else width
    out = np.full((M, width), -np.inf, dtype=np.float64)
    if M == 0 or N == 0 or width == 0:
        return out
    acc = np.zeros((M, N), dtype=np.float64)
    if magnitude:
        q, k, w = np.abs(q), np.abs(k), np.abs(w)
    for h in range(H):
        score = q[:, h, :] @ k.T  # [M, N]
        if k_scale is not None:
            score = score * np.asarray(k_scale, dtype=np.float64)[None, :]
        acc += w[:, h][:, None] * np.maximum(score, 0.0)
    cols = np.arange(min(N, width))
    lo = np.clip(np.asarray(starts, dtype=np.int64), 0, None)
    hi = np.minimum(np.asarray(ends, dtype=np.int64), min(N, width))
    valid = (cols[None, :] >= lo[:, None]) & (cols[None, :] < hi[:, None])
    out[:, : cols.size] = np.where(valid, acc[:, : cols.size], -np.inf)
    return out


def mqa_logits_fp8(q_codes, k_codes, k_scale, w, starts, ends, magnitude: bool = False) -> np.ndarray:
    """Contiguous fp8 chunk: q [M, H, D] e4m3, k [N, D] e4m3 + fp32 scale [N], w [M, H]
    fp32, rows valid on [starts, ends). Returns [M, N] float64."""
    return logits_from_values(
        formats.decode_e4m3(q_codes), formats.decode_e4m3(k_codes), w, starts, ends,
        k_scale=np.asarray(k_scale, dtype=np.float32).reshape(-1), magnitude=magnitude)


# ----------------------------------------------------------------------------------
# paged decode / MTP
# ----------------------------------------------------------------------------------
def paged_row_ends(context_lens, B: int, next_n: int, per_row: bool = False) -> np.ndarray:
    """End (exclusive) of every row r = b * next_n + j of a paged step; start is 0.

    With one length per sequence, row j of a next_n-token verify sees positions
    [0, ctx - next_n + j], its own token included (page
    ``vllm.v1.attention.backends.mla.rocm_aiter_mla``,
    ``AiterMLAHelper.dcp_local_verify_row_lens``), so its end is ctx - next_n + j + 1,
    never below 0. With one length per row (``per_row``) the length is the end.
    """
    cl = np.asarray(context_lens, dtype=np.int64).reshape(-1)
    if per_row:
        return np.maximum(cl[: B * next_n], 0)
    j = np.arange(next_n)
    return np.maximum(cl[:B, None] - next_n + j[None, :] + 1, 0).reshape(-1)


def _paged_keys(pool, fmt: str, P: int, D: int, block_table, b: int, L: int):
    """Dequantised keys 0..L-1 of sequence b: (values [L, D] float64, scale [L] or None)."""
    s = np.arange(L, dtype=np.int64)
    slots = np.asarray(block_table, dtype=np.int64)[b, s // P] * P + s % P
    if fmt == "fp8":
        codes, scales = cache.load_fp8(pool, slots, P, D)
        return formats.decode_e4m3(codes), scales
    packed, sb = cache.load_mxfp4(pool, slots, P, D)
    return formats.decode_mxfp4(packed, sb), None


def paged_logits(pool, fmt: str, P: int, block_table, context_lens, q, w, B: int, next_n: int,
                 width: int, q_scale=None, per_row: bool = False, magnitude: bool = False) -> np.ndarray:
    """Paged decode / MTP logits [B * next_n, width] (page
    ``vllm.v1.attention.ops.rocm_aiter_mla_sparse``, ``rocm_fp8_paged_mqa_logits``; page
    ``vllm.v1.attention.ops.rocm_paged_mxfp4_indexer``, ``rocm_mxfp4_sparse_attn_indexer``).

    fmt "fp8": q [B, next_n, H, D] e4m3, pool pages in the fp8 block-flat layout.
    fmt "mxfp4": q [B, next_n, H, D/2] packed e2m1 with q_scale [B, next_n, H] int32
    (4 e8m0 bytes, byte j for block j), pool pages in the MXFP4 run layout.
    Row r = b * next_n + j is valid on [0, end_r) (``paged_row_ends``), clipped to the
    width and to the keys the block table can address. ``magnitude`` as in
    ``logits_from_values``.
    """
    bt = np.asarray(block_table, dtype=np.int64)
    ends = paged_row_ends(context_lens, B, next_n, per_row)
    H = np.asarray(w).shape[1]
    if fmt == "fp8":
        qv = formats.decode_e4m3(q).reshape(B, next_n, H, -1)
    else:
        qv = formats.decode_mxfp4(q, formats.scales_from_int32(q_scale)).reshape(B, next_n, H, -1)
    D = qv.shape[-1]
    cap = min(width, bt.shape[1] * P)
    out = np.full((B * next_n, width), -np.inf, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    for b in range(B):
        rows = slice(b * next_n, (b + 1) * next_n)
        L = int(min(ends[rows].max(initial=0), cap))
        if L <= 0:
            continue
        kv, ks = _paged_keys(pool, fmt, P, D, bt, b, L)
        out[rows] = logits_from_values(qv[b], kv, w[rows], np.zeros(next_n, np.int64),
                                       np.minimum(ends[rows], L), k_scale=ks, width=width, magnitude=magnitude)
    return out


# ----------------------------------------------------------------------------------
# top-k
# ----------------------------------------------------------------------------------
def topk(logits, starts, ends, k: int) -> np.ndarray:
    """Per-row top-k over columns [start, end) (page
    ``vllm.v1.attention.ops.rocm_paged_mxfp4_indexer``, ``_topk``: rows shorter than k
    are padded with -1).

    The k largest logits are taken, ties at the k-th value going to the lowest column,
    and each is reported as ``column - start`` (a position local to the row's
    sequence). The k chosen indices are listed in ascending column order; a row with
    end <= start is all -1. Ranges are clipped to the logits width.
    """
    L = np.asarray(logits)
    R, W = L.shape
    out = np.full((R, k), -1, dtype=np.int32)
    st = np.clip(np.asarray(starts, dtype=np.int64).reshape(-1), 0, W) if starts is not None else np.zeros(R, np.int64)
    en = np.clip(np.asarray(ends, dtype=np.int64).reshape(-1), 0, W)
    for r in range(R):
        a, b = int(st[r]), int(en[r])
        if b <= a:
            continue
        cols = np.arange(a, b)
        vals = L[r, a:b]
        order = np.lexsort((cols, -vals))  # value descending, then column ascending
        chosen = np.sort(cols[order[:k]])
        out[r, : chosen.size] = (chosen - a).astype(np.int32)
    return out


def topk_to_slots(topk_idx, row_seq, block_table, page_size: int, row_valid=None):
    """Top-k rows of local key positions -> a ragged stream of physical cache slots
    (page ``vllm.v1.attention.ops.rocm_aiter_mla_sparse``,
    ``build_prefill_topk_ragged_indices``: top-k rows hold positions local to each
    sequence, mapped through the sequence's block table to compressed-cache slots and
    packed row after row; page ``vllm.models.deepseek_v41.amd.rocm``,
    ``_decode_topk_ragged``: the decode rows take the same mapping with the
    request of each token and its validity flag).

    Position p of row r (sequence b = row_seq[r]) is slot
    block_table[b, p // page_size] * page_size + p % page_size. Entries < 0 (the -1
    pads) and positions past the block table are dropped, as are all entries of a row
    whose valid flag is 0. Returns (slots [total] int32, indptr [rows + 1] int32,
    lens [rows] int32), the slots of row r at slots[indptr[r]:indptr[r + 1]] in the
    order of the row's entries.
    """
    topk_idx = np.asarray(topk_idx)
    rows, k = topk_idx.shape
    bt = np.asarray(block_table)
    max_blocks = bt.shape[1]
    out, lens = [], np.zeros(rows, dtype=np.int32)
    for r in range(rows):
        if row_valid is not None and not row_valid[r]:
            continue
        b = int(row_seq[r])
        for p in topk_idx[r]:
            p = int(p)
            if p < 0 or p >= max_blocks * page_size:
                continue
            out.append(int(bt[b, p // page_size]) * page_size + p % page_size)
            lens[r] += 1
    indptr = np.zeros(rows + 1, dtype=np.int32)
    indptr[1:] = np.cumsum(lens)
    return np.array(out, dtype=np.int32), indptr, lens
