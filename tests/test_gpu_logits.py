"""GPU parity of the logits calls against the oracle on small seeded inputs that span
several tiles, ragged tails and the degenerate cases (empty rows, rows shorter than a
chunk, zero-length sequences, non-64 page sizes, padded page strides, MTP rows)."""

import numpy as np
import pytest
import torch

from oracle import indexer
from sparse_attention_indexer_mxfp4_amd import ops, workloads
from tests import _inputs, _parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _run_contig(ci, starts, ends):
    wl = ci.wl
    out = ops.idx_mqa_logits(_dev(ci.q), _dev(ci.k), _dev(ci.k_scale), _dev(wl.w), _dev(starts.astype(np.int32)),
                             _dev(ends.astype(np.int32)))
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("M,N,H", [(4, 256, 4), (37, 301, 64), (9, 1000, 16), (64, 130, 24), (3, 64, 128),
                                   (17, 65, 1)])
def test_mqa_logits_random(M, N, H):
    rng = np.random.default_rng(M * 1000 + N + H)
    starts = rng.integers(0, N // 3 + 1, M)
    ends = rng.integers(0, N + 1, M)
    ends[0] = N  # one full row
    if M > 2:
        starts[1], ends[1] = 5, 5  # an empty row
        starts[2], ends[2] = 0, 1  # a single key
    wl = workloads.contiguous(seed=M + N, M=M, N=N, H=H, starts=starts, ends=ends)
    ci = _inputs.contig_inputs(wl)
    got = _run_contig(ci, wl.ks, wl.ke)
    want = indexer.mqa_logits_fp8(ci.q, ci.k, ci.k_scale, wl.w, wl.ks, wl.ke)
    mag = indexer.mqa_logits_fp8(ci.q, ci.k, ci.k_scale, wl.w, wl.ks, wl.ke, magnitude=True)
    _parity.check_logits(got, want, mag, what=f"mqa M={M} N={N} H={H}")


def test_mqa_logits_causal_tiles():
    wl = workloads.contiguous(seed=5, M=300, N=300, H=64, causal_offset=0)
    ci = _inputs.contig_inputs(wl)
    got = _run_contig(ci, wl.ks, wl.ke)
    want = indexer.mqa_logits_fp8(ci.q, ci.k, ci.k_scale, wl.w, wl.ks, wl.ke)
    _parity.check_logits(got, want, what="causal 300", allow_floor=False)


def test_mqa_logits_many_tiles():
    # more row tiles than three rounds of resident workgroups: each workgroup scores
    # several tiles in snake order; every row is compared
    M, N = 12300, 200
    rng = np.random.default_rng(77)
    starts = rng.integers(0, 40, M)
    ends = np.minimum(N, np.arange(M) % (N + 7))
    wl = workloads.contiguous(seed=78, M=M, N=N, H=8, starts=starts, ends=ends)
    ci = _inputs.contig_inputs(wl)
    got = _run_contig(ci, wl.ks, wl.ke)
    want = indexer.mqa_logits_fp8(ci.q, ci.k, ci.k_scale, wl.w, wl.ks, wl.ke)
    mag = indexer.mqa_logits_fp8(ci.q, ci.k, ci.k_scale, wl.w, wl.ks, wl.ke, magnitude=True)
    _parity.check_logits(got, want, mag, what=f"mqa M={M} N={N}")


def test_mqa_logits_config1():
    wl = workloads.config1()
    ci = _inputs.contig_inputs(wl)
    got = _run_contig(ci, wl.ks, wl.ke)
    want = indexer.mqa_logits_fp8(ci.q, ci.k, ci.k_scale, wl.w, wl.ks, wl.ke)
    _parity.check_logits(got, want, what="config 1", allow_floor=False)
    # the whole indexer step: logits then top-k
    idx = ops.idx_topk(_dev(got.astype(np.float32)), _dev(wl.ks), _dev(wl.ke), wl.topk).cpu().numpy()
    _parity.check_topk(idx, indexer.topk(want, wl.ks, wl.ke, wl.topk), want, wl.ks, what="config 1 top-k")


def _run_paged(pi, ctx=None, per_row=False, width=None):
    wl = pi.wl
    fmt = ops.FP8 if wl.fmt == "fp8" else ops.MXFP4
    ctx = wl.context_lens if ctx is None else ctx
    logits, ends = ops.idx_paged_mqa_logits(
        _dev(pi.pool), fmt, wl.page_size, _dev(pi.q), None if pi.q_scale is None else _dev(pi.q_scale), _dev(wl.w),
        _dev(ctx.astype(np.int32)), _dev(wl.block_table), wl.width if width is None else width, ctx_per_row=per_row)
    torch.cuda.synchronize()
    return logits.cpu().numpy(), ends.cpu().numpy()


def _oracle_paged(pi, ctx=None, per_row=False, width=None, magnitude=False):
    wl = pi.wl
    ctx = wl.context_lens if ctx is None else ctx
    return indexer.paged_logits(pi.pool, wl.fmt, wl.page_size, wl.block_table, ctx, pi.q, wl.w, wl.B, wl.next_n,
                                wl.width if width is None else width, q_scale=pi.q_scale, per_row=per_row,
                                magnitude=magnitude)


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("next_n", [1, 2, 3, 4])
def test_paged_random(fmt, next_n):
    lens = np.array([0, 1, 63, 64, 65, 200, 1000, 3, 513])
    wl = workloads.paged(seed=7 + next_n, B=len(lens), next_n=next_n, H=64, ctx_lo=0, ctx_hi=0, width=1100, topk=64,
                         fmt=fmt, context_lens=lens)
    pi = _inputs.paged_inputs(wl, stride_pad=32)
    got, ends = _run_paged(pi)
    want = _oracle_paged(pi)
    np.testing.assert_array_equal(ends, indexer.paged_row_ends(wl.context_lens, wl.B, wl.next_n).clip(0, wl.width))
    _parity.check_logits(got, want, _oracle_paged(pi, magnitude=True), what=f"paged {fmt} next_n={next_n}")


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("page_size,H", [(16, 64), (128, 32), (64, 16), (32, 128)])
def test_paged_page_sizes_and_heads(fmt, page_size, H):
    lens = np.array([5, 130, 700, 64, 1])
    wl = workloads.paged(seed=page_size + H, B=len(lens), next_n=2, H=H, ctx_lo=0, ctx_hi=0, width=770, topk=32,
                         fmt=fmt, context_lens=lens, page_size=page_size)
    pi = _inputs.paged_inputs(wl)
    got, _ = _run_paged(pi)
    _parity.check_logits(got, _oracle_paged(pi), _oracle_paged(pi, magnitude=True),
                         what=f"paged {fmt} P={page_size} H={H}")


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("H", [7, 32, 40, 128])
def test_paged_single_row_heads(fmt, H):
    # one row per sequence with one, two, three (of four) and eight 16-head tiles: the
    # walk's single-row instantiations, each with its own occupancy and workgroup size
    lens = np.array([5, 130, 700, 64, 1, 0, 1000, 257])
    wl = workloads.paged(seed=500 + H, B=len(lens), next_n=1, H=H, ctx_lo=0, ctx_hi=0, width=1030, topk=32,
                         fmt=fmt, context_lens=lens)
    pi = _inputs.paged_inputs(wl, stride_pad=16)
    got, ends = _run_paged(pi)
    np.testing.assert_array_equal(ends, np.minimum(lens, wl.width))
    _parity.check_logits(got, _oracle_paged(pi), _oracle_paged(pi, magnitude=True),
                         what=f"paged {fmt} next_n=1 H={H}")


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_paged_per_row_lengths_and_clamping(fmt):
    lens = np.array([300, 40, 129])
    wl = workloads.paged(seed=3, B=3, next_n=2, H=64, ctx_lo=0, ctx_hi=0, width=320, topk=16, fmt=fmt,
                         context_lens=lens)
    pi = _inputs.paged_inputs(wl)
    per_row = np.array([300, 10, 0, 40, 129, 5000])  # 5000 is clamped to the block table's reach
    got, ends = _run_paged(pi, ctx=per_row, per_row=True)
    want = _oracle_paged(pi, ctx=per_row, per_row=True)
    np.testing.assert_array_equal(ends, np.minimum(per_row, wl.max_blocks * wl.page_size))
    mag = _oracle_paged(pi, ctx=per_row, per_row=True, magnitude=True)
    _parity.check_logits(got, want, mag, what=f"paged {fmt} per-row")


def test_paged_narrow_width():
    # a width below the context truncates every row at the width
    lens = np.array([500, 90])
    wl = workloads.paged(seed=4, B=2, next_n=1, H=64, ctx_lo=0, ctx_hi=0, width=512, topk=16, fmt="fp8",
                         context_lens=lens)
    pi = _inputs.paged_inputs(wl)
    got, ends = _run_paged(pi, width=130)
    want = _oracle_paged(pi, width=130)
    assert ends.tolist() == [130, 90]
    _parity.check_logits(got, want, _oracle_paged(pi, width=130, magnitude=True), what="narrow width")
