"""GPU parity of the two-level indexer (block maxima from the source walk, the candidate
pool, the masked and gathered consumers, the remap of pool slots) against the oracle.

Everything past the logits is selection over given floats, so each step is checked
bit for bit against the oracle applied to the GPU's own inputs to that step; the
gathered pool logits are the dense walk's logits at the gathered positions, bit for
bit, and both sit within the logits tolerance of the oracle's exact values."""

import numpy as np
import pytest
import torch

from oracle import candidates, indexer
from sparse_attention_indexer_mxfp4_amd import ops, workloads
from tests import _inputs, _parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _workload(fmt, next_n, seed, lens=None, width=1600, H=64, page_size=64):
    if lens is None:
        lens = np.array([0, 1, 15, 16, 17, 63, 64, 65, 200, 1000, 1500, 3, 513, 1200])
    wl = workloads.paged(seed=seed, B=len(lens), next_n=next_n, H=H, ctx_lo=0, ctx_hi=0, width=width, topk=64,
                         fmt=fmt, context_lens=lens, page_size=page_size)
    return wl, _inputs.paged_inputs(wl, stride_pad=32)


def _args(pi):
    wl = pi.wl
    fmt = ops.FP8 if wl.fmt == "fp8" else ops.MXFP4
    return (_dev(pi.pool), fmt, wl.page_size, _dev(pi.q), None if pi.q_scale is None else _dev(pi.q_scale),
            _dev(wl.w), _dev(wl.context_lens.astype(np.int32)), _dev(wl.block_table))


def _source(pi, block):
    wl = pi.wl
    logits, ends, bm = ops.idx_paged_mqa_logits_block_max(*_args(pi), wl.width, block)
    return logits, ends, bm


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("next_n", [1, 2, 4])
@pytest.mark.parametrize("block", [16, 32, 64])
def test_block_max_source(fmt, next_n, block):
    wl, pi = _workload(fmt, next_n, seed=40 + next_n + block)
    logits, ends, bm = _source(pi, block)
    plain, plain_ends = ops.idx_paged_mqa_logits(*_args(pi), wl.width)
    torch.cuda.synchronize()
    L = logits.cpu().numpy()
    # the source walk writes the same logits as the plain walk
    np.testing.assert_array_equal(L, plain.cpu().numpy())
    np.testing.assert_array_equal(ends.cpu().numpy(), plain_ends.cpu().numpy())
    e = ends.cpu().numpy()
    # block maxima of its own logits, bit for bit
    np.testing.assert_array_equal(bm.cpu().numpy(), candidates.block_scores(L, e, block).astype(np.float32))
    if next_n == 1 and block == 32:
        want = indexer.paged_logits(pi.pool, wl.fmt, wl.page_size, wl.block_table, wl.context_lens, pi.q, wl.w, wl.B,
                                    wl.next_n, wl.width, q_scale=pi.q_scale)
        _parity.check_logits(L, want, what=f"source {fmt}")


@pytest.mark.parametrize("block,n", [(16, 1), (16, 40), (64, 8), (32, 100)])
def test_candidate_blocks(block, n):
    wl, pi = _workload("fp8", 2, seed=50 + block)
    _, ends, bm = _source(pi, block)
    cand = ops.idx_candidate_blocks(bm, ends, block, n).cpu().numpy()
    want = candidates.candidate_blocks(bm.cpu().numpy(), ends.cpu().numpy(), block, n)
    np.testing.assert_array_equal(cand, want)


def test_candidate_blocks_with_ties():
    # integer-valued block scores: many equal values, ties go to the lower block
    rng = np.random.default_rng(60)
    rows, nb, block, n = 37, 300, 16, 24
    bm = rng.integers(-4, 5, (rows, nb)).astype(np.float32)
    ends = rng.integers(0, nb * block + 1, rows).astype(np.int32)
    ends[:3] = [0, 1, nb * block]
    cand = ops.idx_candidate_blocks(_dev(bm), _dev(ends), block, n).cpu().numpy()
    np.testing.assert_array_equal(cand, candidates.candidate_blocks(bm, ends, block, n))


@pytest.mark.parametrize("row_repeat", [1, 2])
@pytest.mark.parametrize("block", [1, 4, 16, 64])
def test_candidate_mask(row_repeat, block):
    rng = np.random.default_rng(70 + block + row_repeat)
    rows, width, n = 12, 1037, 9
    L = rng.standard_normal((rows, width)).astype(np.float32)
    ends = rng.integers(0, width + 1, rows).astype(np.int32)
    ends[:2] = [0, width]
    nb = -(-width // block)
    # any list: unsorted, repeated, -1 and out-of-range entries
    cand = rng.integers(-1, nb + 3, (rows // row_repeat, n)).astype(np.int32)
    t = torch.empty((rows, (width + 3) // 4 * 4), dtype=torch.float32, device=DEV)[:, :width]
    t.copy_(_dev(L))
    ops.idx_apply_candidate_mask(t, _dev(ends), _dev(cand), block, row_repeat)
    want = candidates.candidate_mask(L, ends, cand, block, row_repeat)
    # columns at or past the end are left as they were
    for r in range(rows):
        want[r, ends[r]:] = L[r, ends[r]:]
    np.testing.assert_array_equal(t.cpu().numpy(), want.astype(np.float32))


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("next_n,row_repeat", [(1, 1), (2, 1), (2, 2), (3, 3)])
@pytest.mark.parametrize("block,n", [(16, 20), (64, 6), (32, 1)])
def test_gather_consumer(fmt, next_n, row_repeat, block, n):
    wl, pi = _workload(fmt, next_n, seed=80 + 7 * next_n + block + n)
    dense, ends, bm = _source(pi, block)
    cand = ops.idx_candidate_blocks(bm, ends, block, n)
    if row_repeat > 1:
        cand = cand[row_repeat - 1::row_repeat].contiguous()  # the last row of each group picks
    pool, pool_end = ops.idx_paged_mqa_logits_gather(*_args(pi), cand, block, row_repeat)
    torch.cuda.synchronize()
    D, e, c = dense.cpu().numpy(), ends.cpu().numpy(), cand.cpu().numpy()
    got = pool.cpu().numpy()
    # the dense walk's logits at the gathered positions, bit for bit
    np.testing.assert_array_equal(got, candidates.gather_logits(D, e, c, block, row_repeat).astype(np.float32))
    np.testing.assert_array_equal(pool_end.cpu().numpy(), candidates.gather_row_ends(c, e, block, wl.rows, row_repeat))
    if block == 16 and next_n == 2:
        want = indexer.paged_logits(pi.pool, wl.fmt, wl.page_size, wl.block_table, wl.context_lens, pi.q, wl.w, wl.B,
                                    wl.next_n, wl.width, q_scale=pi.q_scale)
        _parity.check_logits(got, candidates.gather_logits(want, e, c, block, row_repeat), what=f"gather {fmt}")


def test_gather_any_list_and_page_sizes():
    # unsorted lists with -1 holes and blocks past the end; page size 16 with 16-key blocks
    # and page size 128 with 128-key blocks
    rng = np.random.default_rng(90)
    for page_size, block in ((16, 16), (128, 128), (32, 64)):
        wl, pi = _workload("mxfp4", 2, seed=91 + page_size, width=1664, H=32, page_size=page_size)
        dense, ends = ops.idx_paged_mqa_logits(*_args(pi), wl.width)
        nb = -(-wl.width // block)
        cand = rng.integers(-1, nb + 2, (wl.rows, 11)).astype(np.int32)
        pool, pool_end = ops.idx_paged_mqa_logits_gather(*_args(pi), _dev(cand), block)
        torch.cuda.synchronize()
        D, e = dense.cpu().numpy(), ends.cpu().numpy()
        np.testing.assert_array_equal(pool.cpu().numpy(), candidates.gather_logits(D, e, cand, block).astype(np.float32))
        np.testing.assert_array_equal(pool_end.cpu().numpy(), candidates.gather_row_ends(cand, e, block, wl.rows))


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("H", [7, 32, 40, 128])
def test_gather_heads(fmt, H):
    # the gathered walk's instantiations for one, two, three (of four) and eight head
    # tiles: bit for bit the dense walk's logits at the gathered positions
    block, n = 32, 9
    wl, pi = _workload(fmt, 1, seed=600 + H, H=H)
    dense, ends, bm = _source(pi, block)
    cand = ops.idx_candidate_blocks(bm, ends, block, n)
    pool, pool_end = ops.idx_paged_mqa_logits_gather(*_args(pi), cand, block)
    torch.cuda.synchronize()
    D, e, c = dense.cpu().numpy(), ends.cpu().numpy(), cand.cpu().numpy()
    np.testing.assert_array_equal(pool.cpu().numpy(), candidates.gather_logits(D, e, c, block).astype(np.float32))
    np.testing.assert_array_equal(pool_end.cpu().numpy(), candidates.gather_row_ends(c, e, block, wl.rows))


@pytest.mark.parametrize("row_repeat", [1, 3])
def test_remap(row_repeat):
    rng = np.random.default_rng(100 + row_repeat)
    rows, k, n, block = 30, 50, 12, 32
    cand = rng.integers(-1, 400, (rows // row_repeat, n)).astype(np.int32)
    t = rng.integers(-1, n * block + 40, (rows, k)).astype(np.int32)  # entries past the list too
    got = ops.idx_remap_compact_topk(_dev(t), _dev(cand), block, row_repeat).cpu().numpy()
    np.testing.assert_array_equal(got, candidates.remap_compact_topk(t, cand, block, row_repeat))


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_two_level_step(fmt):
    # source -> pool -> gathered consumer -> top-k over the pool -> remap, against the
    # masked route on the same logits and against the oracle's whole chain
    wl, pi = _workload(fmt, 2, seed=110, lens=np.array([1500, 900, 64, 1300, 5, 700]))
    block, n, k = 16, 24, 100
    dense, ends, bm = _source(pi, block)
    cand = ops.idx_candidate_blocks(bm, ends, block, n)
    pool, pool_end = ops.idx_paged_mqa_logits_gather(*_args(pi), cand, block)
    tk = ops.idx_remap_compact_topk(ops.idx_topk(pool, None, pool_end, k), cand, block)
    masked = ops.idx_apply_candidate_mask(dense.clone(), ends, cand, block)
    tk_masked = ops.idx_topk(masked, None, ends, k)
    torch.cuda.synchronize()
    e = ends.cpu().numpy()
    c = cand.cpu().numpy()
    valid = np.array([candidates.gather_row_ends(c, e, block, wl.rows)[r] >= k for r in range(wl.rows)])
    got, got_m = tk.cpu().numpy(), tk_masked.cpu().numpy()
    # where the pool holds at least k positions both routes select the same positions
    np.testing.assert_array_equal(got[valid], got_m[valid])
    # the oracle's chain over the same pool on its exact logits (the pool itself is
    # checked bit for bit against the oracle's choice from these block maxima above)
    want = indexer.paged_logits(pi.pool, wl.fmt, wl.page_size, wl.block_table, wl.context_lens, pi.q, wl.w, wl.B,
                                wl.next_n, wl.width, q_scale=pi.q_scale)
    pe = candidates.gather_row_ends(c, e, block, wl.rows)
    ow = candidates.remap_compact_topk(indexer.topk(candidates.gather_logits(want, e, c, block), None, pe, k), c, block)
    _parity.check_topk(got, ow, candidates.candidate_mask(want, e, c, block), np.zeros(wl.rows, np.int64),
                       what=f"two-level {fmt}")


@pytest.mark.parametrize("cfg", [5, 3])
def test_two_level_full_size(cfg):
    # the two-level step of the benchmark (pool of 64 blocks of 64 keys) on the full
    # MXFP4 decode and fp8 MTP workloads: every step bit for bit against the oracle
    # applied to the GPU's own inputs of that step, and the source logits against the
    # oracle's exact ones on sampled whole sequences
    wl = workloads.CONFIGS[cfg]()
    pi = _inputs.paged_inputs(wl)
    block, n, k = 64, 64, wl.topk
    dense, ends, bm = _source(pi, block)
    cand = ops.idx_candidate_blocks(bm, ends, block, n)
    pool, pool_end = ops.idx_paged_mqa_logits_gather(*_args(pi), cand, block)
    tk = ops.idx_remap_compact_topk(ops.idx_topk(pool, None, pool_end, k), cand, block)
    torch.cuda.synchronize()
    D, e, B, c = dense.cpu().numpy(), ends.cpu().numpy(), bm.cpu().numpy(), cand.cpu().numpy()
    np.testing.assert_array_equal(B, candidates.block_scores(D, e, block).astype(np.float32))
    np.testing.assert_array_equal(c, candidates.candidate_blocks(B, e, block, n))
    P = pool.cpu().numpy()
    np.testing.assert_array_equal(P, candidates.gather_logits(D, e, c, block).astype(np.float32))
    pe = candidates.gather_row_ends(c, e, block, wl.rows)
    np.testing.assert_array_equal(pool_end.cpu().numpy(), pe)
    rows = np.arange(0, wl.rows, max(1, wl.rows // 12))
    got = tk.cpu().numpy()[rows]
    want = candidates.remap_compact_topk(indexer.topk(P[rows].astype(np.float64), None, pe[rows], k), c[rows], block)
    np.testing.assert_array_equal(got, want)
    seqs = sorted(set(int(r) // wl.next_n for r in rows[:4]))
    for b in seqs:
        sub = np.arange(b * wl.next_n, (b + 1) * wl.next_n)
        exact = indexer.paged_logits(pi.pool, wl.fmt, wl.page_size, wl.block_table[b:b + 1], wl.context_lens[b:b + 1],
                                     pi.q[b:b + 1], wl.w[sub], 1, wl.next_n, wl.width,
                                     q_scale=None if pi.q_scale is None else pi.q_scale[b:b + 1])
        _parity.check_logits(D[sub], exact, what=f"config {cfg} source sequence {b}", allow_floor=False)
