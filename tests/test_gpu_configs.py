"""GPU parity at the five measured workloads' full sizes, in the launch configuration
the benchmark times.

All inputs are the seeded synthetic workloads, quantised by the oracle. Every row's
-inf pattern and -1 padding is checked exactly. The paged steps (decode, MTP, MXFP4
decode) compare every row's logits and top-k with the oracle, at the plain 2e-3
bound; the 8192-row prefill chunk compares 260 rows spread over the whole chunk and
over every row position of a workgroup's tile. On the compared rows the GPU top-k
over the GPU logits must also equal the oracle's top-k over the same fp32 logits
exactly.
"""

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


def _check_mask(got, ends, starts=None):
    cols = np.arange(got.shape[1])
    st = np.zeros(got.shape[0], np.int64) if starts is None else np.asarray(starts, np.int64)
    valid = (cols[None, :] >= st[:, None]) & (cols[None, :] < np.asarray(ends, np.int64)[:, None])
    assert np.array_equal(np.isfinite(got), valid), "-inf pattern differs"
    assert not np.isnan(got).any()


def spread_rows(M, tile=8, step=32):
    """About M / step rows spread over [0, M), taking every position of a tile of `tile`
    rows in turn, plus the first two and last two rows."""
    base = np.arange(0, M, step)
    rows = base + np.arange(base.size) % tile
    return np.unique(np.concatenate([rows[rows < M], [0, 1, M - 2, M - 1]]))


def _check_pads(idx, ends, starts, k):
    n = np.clip(np.asarray(ends) - (0 if starts is None else np.asarray(starts)), 0, None)
    want = np.maximum(k - n, 0)
    assert np.array_equal((idx == -1).sum(axis=1), want), "-1 padding differs"


@pytest.mark.parametrize("cfg", [2, 3, 5])
def test_paged_config_full_size(cfg):
    wl = workloads.CONFIGS[cfg]()
    print(f"config {cfg}: {wl.name}, keys {wl.k.shape[0]}", flush=True)
    pi = _inputs.paged_inputs(wl)
    fmt = ops.FP8 if wl.fmt == "fp8" else ops.MXFP4
    logits, ends = ops.idx_paged_mqa_logits(
        _dev(pi.pool), fmt, wl.page_size, _dev(pi.q), None if pi.q_scale is None else _dev(pi.q_scale), _dev(wl.w),
        _dev(wl.context_lens), _dev(wl.block_table), wl.width)
    idx = ops.idx_topk(logits, None, ends, wl.topk)
    torch.cuda.synchronize()
    got, ends, idx = logits.cpu().numpy(), ends.cpu().numpy(), idx.cpu().numpy()
    want_ends = indexer.paged_row_ends(wl.context_lens, wl.B, wl.next_n)
    np.testing.assert_array_equal(ends, want_ends)
    _check_mask(got, ends)
    _check_pads(idx, ends, None, wl.topk)

    # every row of every sequence
    want = indexer.paged_logits(pi.pool, wl.fmt, wl.page_size, wl.block_table, wl.context_lens, pi.q, wl.w, wl.B,
                                wl.next_n, wl.width, q_scale=pi.q_scale)
    print(f"config {cfg}: oracle done ({wl.rows} rows)", flush=True)
    worst = _parity.check_logits(got, want, what=f"config {cfg}", allow_floor=False)
    print(f"config {cfg}: worst logit error {worst:.2e} of the row max (bound 2e-3), all {wl.rows} rows", flush=True)
    _parity.check_topk(idx, indexer.topk(want, None, ends, wl.topk), want, None, what=f"config {cfg}")
    np.testing.assert_array_equal(idx, indexer.topk(got.astype(np.float64), None, ends, wl.topk))


def test_prefill_config4_full_size():
    wl = workloads.config4()
    ci = _inputs.contig_inputs(wl)
    logits = ops.idx_mqa_logits(_dev(ci.q), _dev(ci.k), _dev(ci.k_scale), _dev(wl.w), _dev(wl.ks), _dev(wl.ke))
    idx = ops.idx_topk(logits, _dev(wl.ks), _dev(wl.ke), wl.topk)
    torch.cuda.synchronize()
    got, idx = logits.cpu().numpy(), idx.cpu().numpy()
    _check_mask(got, wl.ke, wl.ks)
    _check_pads(idx, wl.ke, wl.ks, wl.topk)
    rows = spread_rows(wl.M)
    want = indexer.mqa_logits_fp8(ci.q[rows], ci.k, ci.k_scale, wl.w[rows], wl.ks[rows], wl.ke[rows])
    worst = _parity.check_logits(got[rows], want, rows=rows, what="config 4", allow_floor=False)
    print(f"config 4: worst logit error {worst:.2e} of the row max (bound 2e-3), {rows.size} rows", flush=True)
    _parity.check_topk(idx[rows], indexer.topk(want, wl.ks[rows], wl.ke[rows], wl.topk), want, wl.ks[rows],
                       what="config 4")
    np.testing.assert_array_equal(idx[rows], indexer.topk(got[rows].astype(np.float64), wl.ks[rows], wl.ke[rows],
                                                          wl.topk))
