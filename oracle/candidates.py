"""The two-level indexer: block scores from a source layer's logits, the candidate pool
they select, and the two ways a consumer layer uses that pool.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Page ``vllm.v1.attention.ops.rocm_paged_mxfp4_indexer``: the module description says
the candidate source takes its block maxima from the same walk that writes its logits,
and that consumers may walk the candidate pool instead of the whole context, the pool
being resolved once per step; ``reserve_rocm_mxfp4_indexer_workspace`` sizes the block
scores as [rows, ceil(width / block)] fp32; ``rocm_mxfp4_sparse_mqa_indexer`` either
scores only the pool or runs the dense walk masked to the pool;
``_remap_compact_topk`` turns a pool slot j into a context position: j lies in pool
block j // block, which starts at positions[j // block]. Page
``vllm.v1.attention.ops.rocm_aiter_mla_sparse``, ``_apply_candidate_mask_strided``:
masks a row to its candidate blocks over [0, end), with ``row_repeat`` query rows
sharing one candidate row. The pages do not show how the pool is chosen from the block
maxima, nor the bodies of these kernels. Readings taken here:

* block score j of row r: the largest logit of columns [j * block, (j + 1) * block)
  that lie inside [0, end_r); -inf when none does;
* the pool of a row: its n blocks with the largest scores (equal scores go to the
  lower block), listed in ascending block order and padded with -1; that is the
  per-row top-k of the block scores over [0, ceil(end_r / block));
* query row r uses candidate row r // row_repeat;
* masked consumer: I[r, c] stays where c < end_r and block c // block is in the pool;
  every other column is -inf;
* gather consumer: pool slot j of row r holds the logit of position
  cand[j // block] * block + j % block when that candidate is not -1 and the position
  is below end_r, and -inf otherwise; the pool row is n * block wide;
* the pool row's top-k runs over its slots up to the last one that names a position
  (for a list written by ``candidate_blocks`` from the same row ends that is a prefix:
  only the highest candidate can reach past the end); the masked row's top-k runs
  over [0, end). The two routes select the same positions whenever the pool holds at
  least k of the row's positions; below that, the masked route fills up with -inf
  columns outside the pool while the gather route pads with -1;
* remap: a top-k entry j >= 0 over the pool becomes cand[j // block] * block + j % block,
  i.e. the start of its pool block plus the offset; -1 stays -1, and so does an entry
  whose candidate is -1 or that lies past the list (j >= n * block).

All of it is selection and bookkeeping over given logits: no arithmetic beyond max.
"""

from __future__ import annotations

import numpy as np

from . import indexer


def block_scores(logits, ends, block: int) -> np.ndarray:
    """[rows, ceil(width / block)] float: the largest logit of each block inside the
    row's [0, end), -inf for blocks with no such column."""
    L = np.asarray(logits, dtype=np.float64)
    R, W = L.shape
    nb = -(-W // block)
    out = np.full((R, nb), -np.inf)
    en = np.clip(np.asarray(ends, dtype=np.int64).reshape(-1), 0, W)
    for r in range(R):
        for j in range(nb):
            lo, hi = j * block, min((j + 1) * block, int(en[r]))
            if lo < hi:
                out[r, j] = np.max(L[r, lo:hi])
    return out


def candidate_blocks(scores, ends, block: int, n: int) -> np.ndarray:
    """[rows, n] int32: the n best blocks of each row, ascending, -1 padded."""
    en = np.asarray(ends, dtype=np.int64).reshape(-1)
    block_ends = -(-np.maximum(en, 0) // block)
    return indexer.topk(scores, None, block_ends, n)


def candidate_mask(logits, ends, cand, block: int, row_repeat: int = 1) -> np.ndarray:
    """The dense row restricted to the pool: -inf outside [0, end) and outside the
    candidate blocks of the row's candidate row."""
    L = np.asarray(logits, dtype=np.float64)
    R, W = L.shape
    out = np.full_like(L, -np.inf)
    en = np.clip(np.asarray(ends, dtype=np.int64).reshape(-1), 0, W)
    cand = np.asarray(cand)
    for r in range(R):
        for b in cand[r // row_repeat]:
            b = int(b)
            if b < 0:
                continue
            lo, hi = b * block, min((b + 1) * block, int(en[r]))
            if lo < hi:
                out[r, lo:hi] = L[r, lo:hi]
    return out


def gather_positions(cand, ends, block: int, rows: int, row_repeat: int = 1) -> np.ndarray:
    """[rows, n * block] int64: the context position each pool slot names, -1 where the
    candidate is -1 or the position is at or past the row's end."""
    cand = np.asarray(cand)
    n = cand.shape[1]
    en = np.asarray(ends, dtype=np.int64).reshape(-1)
    pos = np.full((rows, n * block), -1, dtype=np.int64)
    for r in range(rows):
        for j in range(n * block):
            b = int(cand[r // row_repeat, j // block])
            p = b * block + j % block
            if b >= 0 and p < en[r]:
                pos[r, j] = p
    return pos


def gather_row_ends(cand, ends, block: int, rows: int, row_repeat: int = 1) -> np.ndarray:
    """[rows] int32: one past the last pool slot of each row that names a position."""
    pos = gather_positions(cand, ends, block, rows, row_repeat)
    out = np.zeros(rows, dtype=np.int32)
    for r in range(rows):
        ok = np.nonzero(pos[r] >= 0)[0]
        if ok.size:
            out[r] = ok[-1] + 1
    return out


def gather_logits(logits, ends, cand, block: int, row_repeat: int = 1) -> np.ndarray:
    """Pool logits [rows, n * block]: the dense logit at each slot's position, -inf on
    empty slots."""
    L = np.asarray(logits, dtype=np.float64)
    pos = gather_positions(cand, ends, block, L.shape[0], row_repeat)
    out = np.full(pos.shape, -np.inf)
    for r in range(L.shape[0]):
        ok = pos[r] >= 0
        out[r, ok] = L[r, pos[r, ok]]
    return out


def remap_compact_topk(topk_idx, cand, block: int, row_repeat: int = 1) -> np.ndarray:
    """Pool-slot top-k entries to context positions (see the module readings)."""
    t = np.asarray(topk_idx)
    cand = np.asarray(cand)
    out = np.full(t.shape, -1, dtype=np.int32)
    for r in range(t.shape[0]):
        for i, j in enumerate(t[r]):
            j = int(j)
            if j < 0 or j // block >= cand.shape[1]:
                continue
            b = int(cand[r // row_repeat, j // block])
            if b >= 0:
                out[r, i] = b * block + j % block
    return out
