"""Python binding of libidx: the C ABI's calls under the same names, taking PyTorch
tensors for device memory and launching on PyTorch's current HIP stream.

Argument marshalling only: every step runs in the library's HIP kernels. Shapes
and dtypes are checked here only as far as needed to hand the right pointers and
sizes over; the library checks everything it can see itself.
"""

from __future__ import annotations

import ctypes

import torch

from . import _abi
from ._abi import IDX_IN_BF16, IDX_IN_F32, IDX_KV_FP8_E4M3, IDX_KV_MXFP4_E2M1, IdxError, PagedCache  # noqa: F401

FP8 = IDX_KV_FP8_E4M3
MXFP4 = IDX_KV_MXFP4_E2M1
HEAD_DIM = 128


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _need(t: torch.Tensor, dtype, name: str, device=None) -> None:
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name}: expected a device tensor")


def _contig(t: torch.Tensor, name: str) -> None:
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_WORKSPACES: dict = {}


def topk_workspace(nbytes: int, device) -> torch.Tensor | None:
    """A zero-filled scratch buffer of at least nbytes for the top-k calls, kept per
    device and reused: the calls leave it zero-filled, as they need it at their start.
    Calls that share it must not overlap (one stream, or ordered streams); a caller that
    runs top-k on several streams at once passes a workspace of its own to each."""
    if nbytes == 0:
        return None
    dev = torch.device(device)
    key = (dev.type, dev.index)
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        _WORKSPACES[key] = ws
    return ws


def page_bytes(fmt: int, page_size: int, head_dim: int = HEAD_DIM) -> int:
    return int(_abi.lib().idx_page_bytes(fmt, page_size, head_dim))


def paged_cache(pool: torch.Tensor, fmt: int, page_size: int, head_dim: int = HEAD_DIM) -> PagedCache:
    """Descriptor of a pool tensor [num_pages, page_stride_bytes] uint8 (page rows may be
    padded beyond the page size)."""
    _need(pool, torch.uint8, "pool")
    if pool.dim() != 2 or pool.stride(1) != 1:
        raise ValueError("pool must be [num_pages, page_stride_bytes] with unit inner stride")
    return PagedCache(fmt=fmt, page_size=page_size, num_pages=pool.shape[0], head_dim=head_dim,
                      page_stride_bytes=pool.stride(0), base=pool.data_ptr())


def idx_mqa_logits(q: torch.Tensor, k: torch.Tensor, k_scale: torch.Tensor, w: torch.Tensor,
                   row_start: torch.Tensor, row_end: torch.Tensor, logits: torch.Tensor | None = None) -> torch.Tensor:
    """Contiguous fp8 logits. q [M, H, 128] uint8 (e4m3 bytes), k [N, 128] uint8, k_scale [N]
    f32, w [M, H] f32, row_start/row_end [M] int32 -> logits [M, N] f32."""
    _need(q, torch.uint8, "q"); _need(k, torch.uint8, "k"); _need(k_scale, torch.float32, "k_scale")
    _need(w, torch.float32, "w"); _need(row_start, torch.int32, "row_start"); _need(row_end, torch.int32, "row_end")
    M, H, D = q.shape
    N = k.shape[0]
    if q.stride(2) != 1 or q.stride(1) != D or k.stride(1) != 1 or w.stride(1) != 1:
        raise ValueError("q heads, k rows and w rows must be dense")
    _contig(k_scale, "k_scale"); _contig(row_start, "row_start"); _contig(row_end, "row_end")
    if logits is None:
        logits = torch.empty((M, (N + 3) // 4 * 4), dtype=torch.float32, device=q.device)[:, :N]
    _need(logits, torch.float32, "logits")
    _abi.check(_abi.lib().idx_mqa_logits(
        _ptr(q), q.stride(0), _ptr(k), k.stride(0), _ptr(k_scale), _ptr(w), w.stride(0), _ptr(row_start),
        _ptr(row_end), M, N, H, D, _ptr(logits), logits.stride(0), _stream()))
    return logits


def _paged_inputs(pool, fmt, page_size, q, q_scale, w, context_lens, block_table):
    cache = paged_cache(pool, fmt, page_size)
    _need(q, torch.uint8, "q"); _need(w, torch.float32, "w"); _need(context_lens, torch.int32, "context_lens")
    _need(block_table, torch.int32, "block_table")
    _contig(q, "q"); _contig(w, "w"); _contig(context_lens, "context_lens")
    if q_scale is not None:
        _need(q_scale, torch.int32, "q_scale"); _contig(q_scale, "q_scale")
    if block_table.stride(1) != 1:
        raise ValueError("block_table rows must be dense")
    return cache


def idx_paged_mqa_logits(pool: torch.Tensor, fmt: int, page_size: int, q: torch.Tensor, q_scale: torch.Tensor | None,
                         w: torch.Tensor, context_lens: torch.Tensor, block_table: torch.Tensor, width: int,
                         ctx_per_row: bool = False, logits: torch.Tensor | None = None,
                         row_end_out: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Paged decode / MTP logits. q [B, next_n, H, 128] (fp8) or [B, next_n, H, 64] (MXFP4) uint8,
    q_scale [B, next_n, H] int32 (MXFP4) or None, w [B*next_n, H] f32, context_lens [B] (or
    [B*next_n] with ctx_per_row) int32, block_table [B, max_blocks] int32.
    Returns (logits [B*next_n, width] f32, row_end [B*next_n] int32)."""
    cache = _paged_inputs(pool, fmt, page_size, q, q_scale, w, context_lens, block_table)
    B, next_n, H = q.shape[:3]
    logits, row_end_out = _paged_outputs(q, B * next_n, width, logits, row_end_out)
    lib = _abi.lib()
    workspace, ws_bytes = _paged_workspace(lib, cache, B, next_n, H, q.device, workspace)
    _abi.check(lib.idx_paged_mqa_logits(
        ctypes.byref(cache), _ptr(q), _ptr(q_scale), _ptr(w), _ptr(context_lens), int(ctx_per_row),
        _ptr(block_table), block_table.stride(0), block_table.shape[1], B, next_n, H, _ptr(logits),
        logits.stride(0), width, _ptr(row_end_out), _ptr(workspace), ws_bytes, _stream()))
    return logits, row_end_out


def _paged_outputs(q, rows, width, logits, row_end_out):
    if logits is None:
        logits = torch.empty((rows, (width + 3) // 4 * 4), dtype=torch.float32, device=q.device)[:, :width]
    if row_end_out is None:
        row_end_out = torch.empty(rows, dtype=torch.int32, device=q.device)
    return logits, row_end_out


def _paged_workspace(lib, cache, B, next_n, H, device, workspace):
    need = lib.idx_paged_mqa_logits_workspace(B, next_n, H, ctypes.byref(cache))
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    return workspace, 0 if workspace is None else workspace.numel() * workspace.element_size()


def idx_paged_mqa_logits_block_max(pool: torch.Tensor, fmt: int, page_size: int, q: torch.Tensor,
                                   q_scale: torch.Tensor | None, w: torch.Tensor, context_lens: torch.Tensor,
                                   block_table: torch.Tensor, width: int, block_size: int, ctx_per_row: bool = False,
                                   logits: torch.Tensor | None = None, row_end_out: torch.Tensor | None = None,
                                   block_max: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """idx_paged_mqa_logits that also returns the block maxima [B*next_n, ceil(width /
    block_size)] f32 (block_size 16, 32 or 64; 0: none, block_max is None).
    Returns (logits, row_end, block_max)."""
    cache = _paged_inputs(pool, fmt, page_size, q, q_scale, w, context_lens, block_table)
    B, next_n, H = q.shape[:3]
    rows = B * next_n
    logits, row_end_out = _paged_outputs(q, rows, width, logits, row_end_out)
    if block_size and block_max is None:
        block_max = torch.empty((rows, -(-width // block_size)), dtype=torch.float32, device=q.device)
    if block_max is not None:
        _need(block_max, torch.float32, "block_max")
        if block_max.stride(1) != 1:
            raise ValueError("block_max rows must be dense")
    lib = _abi.lib()
    workspace, ws_bytes = _paged_workspace(lib, cache, B, next_n, H, q.device, workspace)
    _abi.check(lib.idx_paged_mqa_logits_block_max(
        ctypes.byref(cache), _ptr(q), _ptr(q_scale), _ptr(w), _ptr(context_lens), int(ctx_per_row),
        _ptr(block_table), block_table.stride(0), block_table.shape[1], B, next_n, H, _ptr(logits),
        logits.stride(0), width, _ptr(row_end_out), _ptr(block_max) if block_size else None,
        block_max.stride(0) if block_size else 0, block_size, _ptr(workspace), ws_bytes, _stream()))
    return logits, row_end_out, block_max if block_size else None


def idx_paged_prefill_logits(pool: torch.Tensor, fmt: int, page_size: int, q: torch.Tensor,
                             q_scale: torch.Tensor | None, w: torch.Tensor, row_end: torch.Tensor,
                             block_table_row: torch.Tensor, width: int, logits: torch.Tensor | None = None):
    """A prefill chunk of one sequence off the paged cache: q [M, H, 128] (fp8) or [M, H, 64]
    (MXFP4) uint8, q_scale [M, H] int32 or None, w [M, H] f32, row_end [M] int32,
    block_table_row [max_blocks] int32 -> logits [M, width] f32."""
    cache = _paged_inputs(pool, fmt, page_size, q, q_scale, w, row_end, block_table_row.reshape(1, -1))
    M, H = q.shape[:2]
    if logits is None:
        logits = torch.empty((M, (width + 3) // 4 * 4), dtype=torch.float32, device=q.device)[:, :width]
    _abi.check(_abi.lib().idx_paged_prefill_logits(
        ctypes.byref(cache), _ptr(q), _ptr(q_scale), _ptr(w), _ptr(row_end), _ptr(block_table_row),
        block_table_row.numel(), M, H, _ptr(logits), logits.stride(0), width, _stream()))
    return logits


def _cand_rows(cand: torch.Tensor) -> None:
    _need(cand, torch.int32, "cand")
    if cand.dim() != 2 or cand.stride(1) != 1:
        raise ValueError("cand must be 2-D with dense rows")


def idx_candidate_blocks(block_max: torch.Tensor, row_end: torch.Tensor, block_size: int, n_cand: int,
                         out: torch.Tensor | None = None) -> torch.Tensor:
    """The candidate pool: per row, the n_cand best blocks of block_max [rows, num_blocks]
    f32 within ceil(row_end / block_size), ascending, -1 padded -> [rows, n_cand] int32."""
    _need(block_max, torch.float32, "block_max"); _need(row_end, torch.int32, "row_end")
    _contig(row_end, "row_end")
    if block_max.stride(1) != 1:
        raise ValueError("block_max rows must be dense")
    rows, nb = block_max.shape
    if out is None:
        out = torch.empty((rows, n_cand), dtype=torch.int32, device=block_max.device)
    lib = _abi.lib()
    need = lib.idx_topk_workspace(rows, nb, n_cand)
    workspace = topk_workspace(need, block_max.device)
    _abi.check(lib.idx_candidate_blocks(_ptr(block_max), block_max.stride(0), rows, nb, _ptr(row_end), block_size,
                                        n_cand, _ptr(out), out.stride(0), _ptr(workspace), need, _stream()))
    return out


def idx_apply_candidate_mask(logits: torch.Tensor, row_end: torch.Tensor, cand: torch.Tensor, block_size: int,
                             row_repeat: int = 1) -> torch.Tensor:
    """In place: columns below row_end outside the row's candidate blocks become -inf."""
    _need(logits, torch.float32, "logits"); _need(row_end, torch.int32, "row_end")
    _contig(row_end, "row_end"); _cand_rows(cand)
    if logits.stride(1) != 1:
        raise ValueError("logits rows must be dense")
    rows, width = logits.shape
    _abi.check(_abi.lib().idx_apply_candidate_mask(_ptr(logits), logits.stride(0), rows, width, _ptr(row_end),
                                                   _ptr(cand), cand.stride(0), cand.shape[1], block_size,
                                                   row_repeat, _stream()))
    return logits


def idx_paged_mqa_logits_gather(pool: torch.Tensor, fmt: int, page_size: int, q: torch.Tensor,
                                q_scale: torch.Tensor | None, w: torch.Tensor, context_lens: torch.Tensor,
                                block_table: torch.Tensor, cand: torch.Tensor, block_size: int, row_repeat: int = 1,
                                ctx_per_row: bool = False, pool_logits: torch.Tensor | None = None,
                                pool_end: torch.Tensor | None = None):
    """Score only each row's candidate pool (cand [rows / row_repeat, n_cand] int32).
    Returns (pool_logits [B*next_n, n_cand*block_size] f32, pool_end [B*next_n] int32)."""
    cache = _paged_inputs(pool, fmt, page_size, q, q_scale, w, context_lens, block_table)
    _cand_rows(cand)
    B, next_n, H = q.shape[:3]
    rows = B * next_n
    width = cand.shape[1] * block_size
    if pool_logits is None:
        pool_logits = torch.empty((rows, (width + 3) // 4 * 4), dtype=torch.float32, device=q.device)[:, :width]
    if pool_end is None:
        pool_end = torch.empty(rows, dtype=torch.int32, device=q.device)
    _abi.check(_abi.lib().idx_paged_mqa_logits_gather(
        ctypes.byref(cache), _ptr(q), _ptr(q_scale), _ptr(w), _ptr(context_lens), int(ctx_per_row),
        _ptr(block_table), block_table.stride(0), block_table.shape[1], B, next_n, H, _ptr(cand), cand.stride(0),
        cand.shape[1], block_size, row_repeat, _ptr(pool_logits), pool_logits.stride(0), _ptr(pool_end),
        _stream()))
    return pool_logits, pool_end


def idx_remap_compact_topk(topk: torch.Tensor, cand: torch.Tensor, block_size: int, row_repeat: int = 1):
    """In place: top-k entries over pool slots -> positions (see include/idx.h)."""
    _need(topk, torch.int32, "topk"); _cand_rows(cand)
    if topk.dim() != 2 or topk.stride(1) != 1:
        raise ValueError("topk must be 2-D with dense rows")
    rows, k = topk.shape
    _abi.check(_abi.lib().idx_remap_compact_topk(_ptr(topk), topk.stride(0), rows, k, _ptr(cand), cand.stride(0),
                                                 cand.shape[1], block_size, row_repeat, _stream()))
    return topk


def idx_topk(logits: torch.Tensor, row_start: torch.Tensor | None, row_end: torch.Tensor, k: int,
             out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Per-row top-k over [row_start, row_end) -> [rows, k] int32 (column - start, ascending
    column order, -1 padded). ``workspace``: uint8 device memory of at least
    idx_topk_workspace() bytes, zero-filled before its first use (the call leaves it
    so); by default the per-device buffer of ``topk_workspace``."""
    _need(logits, torch.float32, "logits"); _need(row_end, torch.int32, "row_end")
    _contig(row_end, "row_end")
    if row_start is not None:
        _need(row_start, torch.int32, "row_start"); _contig(row_start, "row_start")
    if logits.stride(1) != 1:
        raise ValueError("logits rows must be dense")
    rows, width = logits.shape
    if out is None:
        out = torch.empty((rows, k), dtype=torch.int32, device=logits.device)
    lib = _abi.lib()
    need = lib.idx_topk_workspace(rows, width, k)
    if workspace is None:
        workspace = topk_workspace(need, logits.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _abi.check(lib.idx_topk(_ptr(logits), logits.stride(0), rows, width, _ptr(row_start), _ptr(row_end), k,
                            _ptr(out), out.stride(0), _ptr(workspace), ws_bytes, _stream()))
    return out


def idx_k_store(pool: torch.Tensor, fmt: int, page_size: int, k: torch.Tensor, slot_mapping: torch.Tensor) -> None:
    """Quantise key rows k [N, 128] (f32 or bf16) into their slots of the pool."""
    cache = paged_cache(pool, fmt, page_size)
    if k.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("k must be float32 or bfloat16")
    _need(slot_mapping, torch.int64, "slot_mapping"); _contig(slot_mapping, "slot_mapping")
    if k.stride(1) != 1:
        raise ValueError("k rows must be dense")
    dt = IDX_IN_F32 if k.dtype == torch.float32 else IDX_IN_BF16
    _abi.check(_abi.lib().idx_k_store(ctypes.byref(cache), _ptr(k), dt, k.stride(0), _ptr(slot_mapping),
                                      k.shape[0], _stream()))


def idx_q_quant(q: torch.Tensor, fmt: int):
    """Quantise query rows q [T, H, 128] (f32 or bf16). fp8 -> ([T, H, 128] uint8, None);
    MXFP4 -> ([T, H, 64] uint8, [T, H] int32)."""
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("q must be float32 or bfloat16")
    T, H, D = q.shape
    if q.stride(2) != 1 or q.stride(1) != D:
        raise ValueError("q heads must be dense")
    dt = IDX_IN_F32 if q.dtype == torch.float32 else IDX_IN_BF16
    if fmt == FP8:
        out = torch.empty((T, H, D), dtype=torch.uint8, device=q.device)
        scale = None
    else:
        out = torch.empty((T, H, D // 2), dtype=torch.uint8, device=q.device)
        scale = torch.empty((T, H), dtype=torch.int32, device=q.device)
    _abi.check(_abi.lib().idx_q_quant(_ptr(q), dt, q.stride(0), T, H, D, fmt, _ptr(out), _ptr(scale), _stream()))
    return out, scale


def _rope_args(positions: torch.Tensor | None, cos_sin: torch.Tensor | None, rope_dim: int):
    if rope_dim == 0:
        return None, None, 1
    if positions is None or cos_sin is None:
        raise ValueError("RoPE needs positions and a cos/sin table")
    _need(positions, torch.int64, "positions"); _contig(positions, "positions")
    _need(cos_sin, torch.float32, "cos_sin"); _contig(cos_sin, "cos_sin")
    if cos_sin.dim() != 2 or cos_sin.shape[1] != rope_dim:
        raise ValueError("cos_sin must be [max_position, rope_dim]")
    return positions, cos_sin, cos_sin.shape[0]


def idx_k_norm_rope_store(pool: torch.Tensor, fmt: int, page_size: int, k: torch.Tensor, slot_mapping: torch.Tensor,
                          positions: torch.Tensor | None, cos_sin: torch.Tensor | None, rope_dim: int,
                          norm_weight: torch.Tensor, eps: float) -> None:
    """RMSNorm (norm_weight [128] f32, eps) and GPT-J RoPE of pre-norm keys k [N, 128]
    (f32 or bf16), then the K store into their slots of the pool."""
    cache = paged_cache(pool, fmt, page_size)
    if k.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("k must be float32 or bfloat16")
    _need(slot_mapping, torch.int64, "slot_mapping"); _contig(slot_mapping, "slot_mapping")
    _need(norm_weight, torch.float32, "norm_weight"); _contig(norm_weight, "norm_weight")
    if k.stride(1) != 1:
        raise ValueError("k rows must be dense")
    pos, cs, maxp = _rope_args(positions, cos_sin, rope_dim)
    dt = IDX_IN_F32 if k.dtype == torch.float32 else IDX_IN_BF16
    _abi.check(_abi.lib().idx_k_norm_rope_store(ctypes.byref(cache), _ptr(k), dt, k.stride(0), _ptr(pos), _ptr(cs),
                                                maxp, rope_dim, _ptr(norm_weight), float(eps), _ptr(slot_mapping),
                                                k.shape[0], _stream()))


def idx_q_rope_quant(q: torch.Tensor, fmt: int, positions: torch.Tensor | None, cos_sin: torch.Tensor | None,
                     rope_dim: int, weights: torch.Tensor, weight_scale: float):
    """GPT-J RoPE of queries q [T, H, 128] (f32 or bf16), quantised as idx_q_quant, and
    weights [T, H] f32 times weight_scale. Returns (q_out, q_scale or None, weights_out)."""
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("q must be float32 or bfloat16")
    T, H, D = q.shape
    if q.stride(2) != 1 or q.stride(1) != D:
        raise ValueError("q heads must be dense")
    _need(weights, torch.float32, "weights")
    if weights.dim() != 2 or tuple(weights.shape) != (T, H) or weights.stride(1) != 1:
        raise ValueError("weights must be [T, H] with dense rows")
    pos, cs, maxp = _rope_args(positions, cos_sin, rope_dim)
    dt = IDX_IN_F32 if q.dtype == torch.float32 else IDX_IN_BF16
    if fmt == FP8:
        out = torch.empty((T, H, D), dtype=torch.uint8, device=q.device)
        scale = None
    else:
        out = torch.empty((T, H, D // 2), dtype=torch.uint8, device=q.device)
        scale = torch.empty((T, H), dtype=torch.int32, device=q.device)
    w_out = torch.empty((T, H), dtype=torch.float32, device=q.device)
    _abi.check(_abi.lib().idx_q_rope_quant(_ptr(q), dt, q.stride(0), _ptr(pos), _ptr(cs), maxp, rope_dim,
                                           _ptr(weights), weights.stride(0), float(weight_scale), T, H, D, fmt,
                                           _ptr(out), _ptr(scale), _ptr(w_out), _stream()))
    return out, scale, w_out


def idx_topk_to_slots(topk: torch.Tensor, block_table: torch.Tensor, page_size: int, next_n: int = 1,
                      row_seq: torch.Tensor | None = None, row_valid: torch.Tensor | None = None,
                      slots: torch.Tensor | None = None, indptr: torch.Tensor | None = None,
                      lens: torch.Tensor | None = None):
    """Top-k rows [rows, k] int32 of local positions -> (slots [rows*k] int32 of which
    the first indptr[-1] are used, indptr [rows + 1] int32, lens [rows] int32). The
    three outputs may be passed in (int32, at least those sizes)."""
    _need(topk, torch.int32, "topk")
    _need(block_table, torch.int32, "block_table")
    if topk.dim() != 2 or topk.stride(1) != 1 or block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("topk and block_table must be 2-D with dense rows")
    if row_seq is not None:
        _need(row_seq, torch.int32, "row_seq"); _contig(row_seq, "row_seq")
    if row_valid is not None:
        _need(row_valid, torch.uint8, "row_valid"); _contig(row_valid, "row_valid")
    rows, k = topk.shape
    dev = topk.device
    if slots is None:
        slots = torch.empty(max(rows * k, 1), dtype=torch.int32, device=dev)
    if indptr is None:
        indptr = torch.empty(rows + 1, dtype=torch.int32, device=dev)
    if lens is None:
        lens = torch.empty(max(rows, 1), dtype=torch.int32, device=dev)
    for t, n, name in ((slots, rows * k, "slots"), (indptr, rows + 1, "indptr"), (lens, rows, "lens")):
        _need(t, torch.int32, name); _contig(t, name)
        if t.numel() < n:
            raise ValueError(f"{name} holds fewer than {n} entries")
    _abi.check(_abi.lib().idx_topk_to_slots(_ptr(topk), topk.stride(0), rows, k, _ptr(row_seq), next_n,
                                            block_table.shape[0], _ptr(row_valid), _ptr(block_table),
                                            block_table.stride(0), block_table.shape[1], page_size, _ptr(slots),
                                            _ptr(indptr), _ptr(lens), _stream()))
    return slots, indptr, lens[:rows]



debug_build = _abi.debug_build  # `with ops.debug_build():` routes the calls to libidx_debug.so


def idx_debug_flags(clear: bool = True) -> int:
    """The IDX_DBG_* bits (_abi.DBG_*) the debug build has recorded on the current device
    since they were last cleared; always 0 for the release build. Waits for the device."""
    out = ctypes.c_uint32(0)
    _abi.check(_abi.lib().idx_debug_flags(ctypes.byref(out), int(clear)))
    return int(out.value)
