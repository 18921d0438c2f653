"""GPU parity of the prefill chunk read straight off the paged cache
(idx_paged_prefill_logits) against the oracle's paged logits with per-row ends: small
cases with ragged row ends, odd row counts, head counts that are not a multiple of 16,
both formats and several page sizes (one not a power of two); the full 8192 x 8192
MXFP4 chunk and a full-size fp8 chunk on 260 rows spread over each; fp8 pages bit for
bit against the contiguous entry point over the same keys laid out contiguously; and,
where the decode walk serves the chunk (MXFP4, 128 heads), every row bit for bit
against the decode entry point fed the same rows as two-row sequences."""

import numpy as np
import pytest
import torch

from oracle import indexer
from sparse_attention_indexer_mxfp4_amd import ops, workloads
from tests import _inputs, _parity
from tests.test_gpu_configs import spread_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _run(pi, row_end=None, width=None):
    wl = pi.wl
    fmt = ops.FP8 if wl.fmt == "fp8" else ops.MXFP4
    re = wl.row_end if row_end is None else row_end
    out = ops.idx_paged_prefill_logits(_dev(pi.pool), fmt, wl.page_size, _dev(pi.q),
                                       None if pi.q_scale is None else _dev(pi.q_scale), _dev(wl.w),
                                       _dev(re.astype(np.int32)), _dev(wl.block_table[0]),
                                       wl.width if width is None else width)
    torch.cuda.synchronize()
    return out


def _oracle(pi, rows, row_end=None, width=None, magnitude=False):
    wl = pi.wl
    re = (wl.row_end if row_end is None else row_end)[rows]
    qs = None if pi.q_scale is None else pi.q_scale[rows][None]
    return indexer.paged_logits(pi.pool, wl.fmt, wl.page_size, wl.block_table, re, pi.q[rows][None], wl.w[rows], 1,
                                len(rows), wl.width if width is None else width, q_scale=qs, per_row=True,
                                magnitude=magnitude)


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("M,N,H,P", [(37, 300, 64, 64), (64, 1000, 16, 16), (130, 777, 32, 128), (3, 200, 64, 64),
                                     (21, 500, 24, 48), (9, 300, 128, 64)])
def test_paged_prefill_small(fmt, M, N, H, P):
    width = -(-N // 64) * 64 + 32
    wl = workloads.paged_prefill(seed=M + N + P, M=M, N=N, H=H, width=width, topk=16, fmt=fmt, page_size=P)
    pi = _inputs.paged_inputs(wl, stride_pad=16)
    got = _run(pi).cpu().numpy()
    rows = np.arange(M)
    _parity.check_logits(got, _oracle(pi, rows), _oracle(pi, rows, magnitude=True), what=f"paged prefill {fmt}")


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_paged_prefill_ragged_ends(fmt):
    # row ends in any order, empty rows, ends past the sequence and past the width
    rng = np.random.default_rng(7)
    wl = workloads.paged_prefill(seed=8, M=45, N=900, H=64, width=1024, topk=16, fmt=fmt)
    pi = _inputs.paged_inputs(wl)
    re = rng.integers(0, 1200, wl.M).astype(np.int32)
    re[:4] = [0, 1, 900, 5000]
    got = _run(pi, row_end=re).cpu().numpy()
    rows = np.arange(wl.M)
    want = _oracle(pi, rows, row_end=re)
    # ends past the sequence's 900 keys reach the rest of its last page and the
    # block-table tail (zero bytes, as the pool was built); both sides read the same
    # bytes, clipped to the table and the width
    _parity.check_logits(got, want, _oracle(pi, rows, row_end=re, magnitude=True), what=f"ragged {fmt}")


def test_paged_prefill_is_the_decode_walk():
    # MXFP4 pages with 128 heads: rows 2g, 2g+1 are one walk of the decode kernel over
    # the same pages, the same bits as idx_paged_mqa_logits with those rows as a two-row
    # (MTP) sequence (fp8 pages and MXFP4 pages with up to 64 heads take the chunk
    # kernels, whose |x| split sums differently)
    fmt = "mxfp4"
    wl = workloads.paged_prefill(seed=9, M=48, N=700, H=128, width=768, topk=16, fmt=fmt)
    pi = _inputs.paged_inputs(wl)
    got = _run(pi).cpu().numpy()
    G = wl.M // 2
    qs = None if pi.q_scale is None else _dev(pi.q_scale.reshape(G, 2, wl.H))
    dec, _ = ops.idx_paged_mqa_logits(_dev(pi.pool), ops.FP8 if fmt == "fp8" else ops.MXFP4, wl.page_size,
                                      _dev(pi.q.reshape((G, 2) + pi.q.shape[1:])), qs, _dev(wl.w),
                                      _dev(wl.row_end), _dev(np.repeat(wl.block_table, G, axis=0)), wl.width,
                                      ctx_per_row=True)
    np.testing.assert_array_equal(got, dec.cpu().numpy())


def test_paged_prefill_full_chunk():
    # the 8192 x 8192 MXFP4 chunk at full size, in the launch the benchmark times:
    # sampled rows against the oracle, and their top-k bit for bit against the
    # oracle's top-k on the GPU's logits
    wl = workloads.config6()
    pi = _inputs.paged_inputs(wl)
    got = _run(pi)
    k = wl.topk
    tk = ops.idx_topk(got, None, _dev(wl.row_end), k).cpu().numpy()
    L = got.cpu().numpy()
    rows = spread_rows(wl.M)
    want = _oracle(pi, rows)
    worst = _parity.check_logits(L[rows], want, what="config 6 spread rows", allow_floor=False)
    print(f"config 6: worst logit error {worst:.2e} of the row max (bound 2e-3), {rows.size} rows", flush=True)
    np.testing.assert_array_equal(tk[rows], indexer.topk(L[rows], None, wl.row_end[rows], k))


def test_paged_prefill_full_chunk_fp8():
    # the 8192 x 8192 chunk on an fp8 paged cache (the contiguous prefill kernel reading
    # its keys through the block table): sampled rows against the oracle, every row's
    # -inf tail
    wl = workloads.paged_prefill(seed=12, M=8192, N=8192, H=64, width=8192, topk=2048, fmt="fp8")
    pi = _inputs.paged_inputs(wl)
    L = _run(pi).cpu().numpy()
    ends = np.minimum(wl.row_end, wl.width)
    cols = np.arange(wl.width)
    assert np.array_equal(np.isneginf(L), cols[None, :] >= ends[:, None])
    rows = spread_rows(wl.M)
    worst = _parity.check_logits(L[rows], _oracle(pi, rows), what="fp8 chunk spread rows", allow_floor=False)
    print(f"fp8 paged chunk: worst logit error {worst:.2e} of the row max (bound 2e-3), {rows.size} rows", flush=True)


@pytest.mark.parametrize("P,pad", [(64, 16), (16, 0), (48, 32)])
def test_paged_prefill_fp8_is_the_contiguous_kernel(P, pad):
    # fp8 pages: the same bits as idx_mqa_logits over the sequence's keys laid out
    # contiguously, since both calls run the one prefill kernel with the same tiling;
    # this pins the page lookups and byte offsets of the paged key reads exactly
    N = 12 * P
    wl = workloads.paged_prefill(seed=20 + P, M=77, N=N, H=64, width=N, topk=16, fmt="fp8", page_size=P)
    pi = _inputs.paged_inputs(wl, stride_pad=pad)
    got = _run(pi).cpu().numpy()
    ends = np.minimum(wl.row_end, N).astype(np.int32)
    contig = ops.idx_mqa_logits(_dev(pi.q), _dev(pi.k_codes[:N]), _dev(pi.k_scales[:N]), _dev(wl.w),
                                _dev(np.zeros(wl.M, np.int32)), _dev(ends))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got, contig.cpu().numpy())


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("M,N,H,width,P", [(1, 50, 1, 57, 16), (5, 130, 7, 130, 64), (9, 1000, 64, 130, 64),
                                           (16, 64, 16, 66, 16)])
def test_paged_prefill_edge_shapes(fmt, M, N, H, width, P):
    # one row and one head, widths that are not a multiple of 4 or of a chunk, a width
    # shorter than the sequence (ends clamped to it), an empty first row
    wl = workloads.paged_prefill(seed=M * 7 + N + width, M=M, N=N, H=H, width=max(width, N), topk=16, fmt=fmt,
                                 page_size=P)
    pi = _inputs.paged_inputs(wl)
    re = wl.row_end.copy()
    re[0] = 0
    got = _run(pi, row_end=re, width=width).cpu().numpy()[:, :width]
    rows = np.arange(M)
    want = _oracle(pi, rows, row_end=np.minimum(re, width), width=width)
    _parity.check_logits(got, want, _oracle(pi, rows, row_end=np.minimum(re, width), width=width, magnitude=True),
                         what=f"edge {fmt} M={M} H={H} width={width}")


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_paged_prefill_empty_block_table(fmt):
    # no block-table entries at all (a NULL table, max_blocks 0) while the rows claim
    # keys: no key exists, so every column of every row is -inf, and nothing may be read
    # through the table or the pool
    wl = workloads.paged_prefill(seed=31, M=64, N=200, H=64, width=512, topk=16, fmt=fmt)
    pi = _inputs.paged_inputs(wl)
    fmt_id = ops.FP8 if fmt == "fp8" else ops.MXFP4
    empty = torch.empty(0, dtype=torch.int32, device=DEV)
    out = ops.idx_paged_prefill_logits(_dev(pi.pool), fmt_id, wl.page_size, _dev(pi.q),
                                       None if pi.q_scale is None else _dev(pi.q_scale), _dev(wl.w),
                                       _dev(np.full(wl.M, 150, np.int32)), empty, wl.width)
    torch.cuda.synchronize()
    assert np.isneginf(out.cpu().numpy()).all()
