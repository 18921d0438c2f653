"""Guard bands around every output: each call writes its outputs and nothing else.

Outputs are views into larger buffers filled with a sentinel bit pattern: rows padded
past their width (the row stride the ABI allows) and one extra row past the last.
Widths are chosen off multiples of 4 and of the 64-key chunk, where the kernels'
16-byte stores and range-checked buffer stores meet the row end. After each call the
padding and the extra row must still hold the sentinel, and the values inside must
equal those of the same call on freshly allocated, unpadded outputs, bit for bit.
"""

import numpy as np
import pytest
import torch

from sparse_attention_indexer_mxfp4_amd import ops, workloads
from tests import _inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SENT = 0x7FC0DEAD  # a NaN payload as float32; never a value any call writes
PAD = 12


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def guarded(rows, cols, dtype=torch.float32):
    """(buffer, view): a [rows, cols] view with a padded row stride (a multiple of 4
    elements) and one spare row, everything filled with the sentinel."""
    stride = -(-cols // 4) * 4 + PAD
    buf = torch.full((rows + 1, stride), SENT, dtype=torch.int32, device=DEV)
    return buf, buf.view(dtype)[:rows, :cols]


def untouched(buf, rows, cols, what):
    b = buf.cpu().numpy()
    assert (b[:rows, cols:] == SENT).all(), f"{what}: padding past a row's width was written"
    assert (b[rows:] == SENT).all(), f"{what}: the row past the last one was written"


def same(got, want, what):
    g = got.contiguous().view(torch.int32).cpu().numpy()
    w = want.contiguous().view(torch.int32).cpu().numpy()
    assert np.array_equal(g, w), f"{what}: values differ from the unpadded call"


def _paged(fmt, next_n=2, H=64):
    # a call may pass a width below the context (rows are cut at the width); the
    # workload itself is drawn at the longest width used here
    lens = np.array([0, 1, 63, 65, 300, 1000, 7])
    wl = workloads.paged(seed=40 + next_n, B=len(lens), next_n=next_n, H=H, ctx_lo=0, ctx_hi=0, width=1101,
                         topk=33, fmt=fmt, context_lens=lens)
    pi = _inputs.paged_inputs(wl, stride_pad=16)
    f = ops.FP8 if fmt == "fp8" else ops.MXFP4
    args = (_dev(pi.pool), f, wl.page_size, _dev(pi.q), None if pi.q_scale is None else _dev(pi.q_scale),
            _dev(wl.w), _dev(wl.context_lens), _dev(wl.block_table))
    return wl, args


def test_guard_mqa_logits():
    M, N, H = 37, 301, 64
    starts = np.arange(M, dtype=np.int32) * 3
    wl = workloads.contiguous(seed=5, M=M, N=N, H=H, starts=starts, ends=np.minimum(starts + 250, N))
    ci = _inputs.contig_inputs(wl)
    args = (_dev(ci.q), _dev(ci.k), _dev(ci.k_scale), _dev(wl.w), _dev(wl.ks), _dev(wl.ke))
    buf, view = guarded(M, N)
    ops.idx_mqa_logits(*args, logits=view)
    want = ops.idx_mqa_logits(*args)
    torch.cuda.synchronize()
    untouched(buf, M, N, "idx_mqa_logits")
    same(view, want, "idx_mqa_logits")


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("next_n,width", [(1, 1101), (2, 1101), (2, 65), (3, 258)])
def test_guard_paged_logits_and_block_max(fmt, next_n, width):
    wl, args = _paged(fmt, next_n)
    rows = wl.rows
    buf, view = guarded(rows, width)
    ebuf, ends = guarded(1, rows, torch.int32)
    ops.idx_paged_mqa_logits(*args, width, logits=view, row_end_out=ends[0])
    want, want_ends = ops.idx_paged_mqa_logits(*args, width)
    torch.cuda.synchronize()
    untouched(buf, rows, width, "idx_paged_mqa_logits")
    untouched(ebuf, 1, rows, "idx_paged_mqa_logits row ends")
    same(view, want, "idx_paged_mqa_logits")
    same(ends[0], want_ends, "idx_paged_mqa_logits row ends")
    nb = -(-width // 32)
    buf2, view2 = guarded(rows, width)
    bbuf, bm = guarded(rows, nb)
    ops.idx_paged_mqa_logits_block_max(*args, width, 32, logits=view2, block_max=bm)
    _, _, want_bm = ops.idx_paged_mqa_logits_block_max(*args, width, 32)
    torch.cuda.synchronize()
    untouched(buf2, rows, width, "idx_paged_mqa_logits_block_max logits")
    untouched(bbuf, rows, nb, "idx_paged_mqa_logits_block_max block maxima")
    same(view2, want, "idx_paged_mqa_logits_block_max logits")
    same(bm, want_bm, "idx_paged_mqa_logits_block_max block maxima")


@pytest.mark.parametrize("fmt,H", [("fp8", 64), ("mxfp4", 64), ("mxfp4", 128)])
def test_guard_paged_prefill(fmt, H):
    M, N, width = 21, 500, 513
    wl = workloads.paged_prefill(seed=M + H, M=M, N=N, H=H, width=width, topk=16, fmt=fmt)
    pi = _inputs.paged_inputs(wl)
    f = ops.FP8 if fmt == "fp8" else ops.MXFP4
    args = (_dev(pi.pool), f, wl.page_size, _dev(pi.q), None if pi.q_scale is None else _dev(pi.q_scale),
            _dev(wl.w), _dev(wl.row_end), _dev(wl.block_table[0]), width)
    buf, view = guarded(M, width)
    ops.idx_paged_prefill_logits(*args, logits=view)
    want = ops.idx_paged_prefill_logits(*args)
    torch.cuda.synchronize()
    untouched(buf, M, width, f"idx_paged_prefill_logits {fmt} H={H}")
    same(view, want, f"idx_paged_prefill_logits {fmt} H={H}")


@pytest.mark.parametrize("rows,width,k", [(5, 1101, 33), (3, 40000, 2048), (1030, 301, 16), (2, 70000, 512)])
def test_guard_topk(rows, width, k):
    rng = np.random.default_rng(rows + width)
    L = rng.standard_normal((rows, width)).astype(np.float32)
    ends = rng.integers(0, width + 1, rows).astype(np.int32)
    ends[0] = width
    starts = np.minimum(rng.integers(0, 50, rows), ends).astype(np.int32)
    lbuf, lv = guarded(rows, width)
    lv.copy_(_dev(L))
    buf, view = guarded(rows, k, torch.int32)
    ops.idx_topk(lv, _dev(starts), _dev(ends), k, out=view)
    want = ops.idx_topk(_dev(L), _dev(starts), _dev(ends), k)
    torch.cuda.synchronize()
    untouched(buf, rows, k, "idx_topk")
    untouched(lbuf, rows, width, "idx_topk input")
    same(view, want, "idx_topk")


def test_guard_topk_to_slots():
    rng = np.random.default_rng(3)
    rows, k, B, P, mb = 9, 40, 3, 16, 8
    topk = rng.integers(-1, mb * P + 5, (rows, k)).astype(np.int32)
    bt = rng.permutation(B * mb).reshape(B, mb).astype(np.int32)
    tbuf, tv = guarded(rows, k, torch.int32)
    tv.copy_(_dev(topk))
    slots = torch.full((rows * k + 64,), SENT, dtype=torch.int32, device=DEV)
    indptr = torch.full((rows + 1 + 8,), SENT, dtype=torch.int32, device=DEV)
    lens = torch.full((rows + 8,), SENT, dtype=torch.int32, device=DEV)
    ops.idx_topk_to_slots(tv, _dev(bt), P, next_n=3, slots=slots, indptr=indptr, lens=lens)
    ws, wi, wlens = ops.idx_topk_to_slots(_dev(topk), _dev(bt), P, next_n=3)
    torch.cuda.synchronize()
    s, ip, ln = slots.cpu().numpy(), indptr.cpu().numpy(), lens.cpu().numpy()
    total = int(ip[rows])
    assert (s[total:] == SENT).all(), "slots past the last used entry were written"
    assert (ip[rows + 1:] == SENT).all() and (ln[rows:] == SENT).all()
    assert np.array_equal(ip[:rows + 1], wi.cpu().numpy()) and np.array_equal(ln[:rows], wlens.cpu().numpy())
    assert np.array_equal(s[:total], ws.cpu().numpy()[:total])
    untouched(tbuf, rows, k, "idx_topk_to_slots input")


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_guard_two_level(fmt):
    width, block, n_cand, k = 1101, 32, 7, 40
    wl, args = _paged(fmt, 2)
    rows = wl.rows
    logits, ends, bm = ops.idx_paged_mqa_logits_block_max(*args, width, block)
    # the pool: guarded output, then unpadded
    cbuf, cand = guarded(rows, n_cand, torch.int32)
    ops.idx_candidate_blocks(bm, ends, block, n_cand, out=cand)
    want_cand = ops.idx_candidate_blocks(bm, ends, block, n_cand)
    torch.cuda.synchronize()
    untouched(cbuf, rows, n_cand, "idx_candidate_blocks")
    same(cand, want_cand, "idx_candidate_blocks")
    # masked consumer, in place on a padded copy of the dense logits
    mbuf, masked = guarded(rows, width)
    masked.copy_(logits)
    ops.idx_apply_candidate_mask(masked, ends, cand, block)
    fresh = torch.empty((rows, -(-width // 4) * 4), dtype=torch.float32, device=DEV)[:, :width]
    fresh.copy_(logits)
    want_masked = ops.idx_apply_candidate_mask(fresh, ends, want_cand, block)
    torch.cuda.synchronize()
    untouched(mbuf, rows, width, "idx_apply_candidate_mask")
    same(masked, want_masked, "idx_apply_candidate_mask")
    # gathered consumer
    pw = n_cand * block
    pbuf, pool_logits = guarded(rows, pw)
    ebuf, pend = guarded(1, rows, torch.int32)
    ops.idx_paged_mqa_logits_gather(*args, cand, block, pool_logits=pool_logits, pool_end=pend[0])
    want_pool, want_pend = ops.idx_paged_mqa_logits_gather(*args, want_cand, block)
    torch.cuda.synchronize()
    untouched(pbuf, rows, pw, "idx_paged_mqa_logits_gather")
    untouched(ebuf, 1, rows, "idx_paged_mqa_logits_gather pool ends")
    same(pool_logits, want_pool, "idx_paged_mqa_logits_gather")
    same(pend[0], want_pend, "idx_paged_mqa_logits_gather pool ends")
    # remap, in place on a padded top-k
    tk = ops.idx_topk(want_pool, None, want_pend, k)
    rbuf, rv = guarded(rows, k, torch.int32)
    rv.copy_(tk)
    ops.idx_remap_compact_topk(rv, cand, block)
    want_r = ops.idx_remap_compact_topk(tk.clone(), want_cand, block)
    torch.cuda.synchronize()
    untouched(rbuf, rows, k, "idx_remap_compact_topk")
    same(rv, want_r, "idx_remap_compact_topk")
