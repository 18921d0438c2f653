"""Pins of the two-level indexer oracle (oracle/candidates.py) against a hand-worked
step, brute force on tiny inputs, and the special cases where it reduces to the dense
indexer."""

import json
import os

import numpy as np

from oracle import candidates, indexer

HERE = os.path.dirname(__file__)


def _arr(x):
    return np.array([[float(v) for v in row] for row in x])


def test_handworked_two_level_step():
    g = json.load(open(os.path.join(HERE, "golden", "handworked_two_level.json")))
    L, ends, block, n, k = _arr(g["logits"]), np.array(g["ends"]), g["block"], g["n"], g["k"]
    bs = candidates.block_scores(L, ends, block)
    np.testing.assert_array_equal(bs, _arr(g["block_scores"]))
    cand = candidates.candidate_blocks(bs, ends, block, n)
    np.testing.assert_array_equal(cand, g["cand"])
    masked = candidates.candidate_mask(L, ends, cand, block)
    np.testing.assert_array_equal(masked, _arr(g["masked"]))
    pool = candidates.gather_logits(L, ends, cand, block)
    np.testing.assert_array_equal(pool, _arr(g["pool"]))
    pool_ends = candidates.gather_row_ends(cand, ends, block, L.shape[0])
    np.testing.assert_array_equal(pool_ends, g["pool_ends"])
    ptk = indexer.topk(pool, None, pool_ends, k)
    np.testing.assert_array_equal(ptk, g["pool_topk"])
    np.testing.assert_array_equal(candidates.remap_compact_topk(ptk, cand, block), g["positions"])
    np.testing.assert_array_equal(indexer.topk(masked, None, ends, k), g["masked_topk"])


def _random_step(rng, rows, width, ties=False):
    if ties:
        L = rng.integers(-3, 4, (rows, width)).astype(np.float64)
    else:
        L = rng.standard_normal((rows, width))
    ends = rng.integers(0, width + 1, rows)
    ends[0] = width
    return L, ends


def test_block_scores_brute_force():
    # each score is attained inside its block and bounds every column of the block
    # below the row end; blocks with no such column are -inf
    rng = np.random.default_rng(1)
    for block in (1, 3, 4, 16):
        L, ends = _random_step(rng, 5, 50)
        bs = candidates.block_scores(L, ends, block)
        assert bs.shape == (5, -(-50 // block))
        for r in range(5):
            for j in range(bs.shape[1]):
                cols = [c for c in range(j * block, min((j + 1) * block, 50)) if c < ends[r]]
                if not cols:
                    assert bs[r, j] == -np.inf
                else:
                    assert bs[r, j] in L[r, cols] and all(bs[r, j] >= L[r, c] for c in cols)


def test_pool_covering_the_row_is_the_dense_indexer():
    # with n * block >= end every block in range is a candidate: the masked row is the
    # dense row and both routes give the dense top-k
    rng = np.random.default_rng(2)
    for ties in (False, True):
        L, ends = _random_step(rng, 6, 64, ties)
        block, k = 8, 10
        n = 8
        bs = candidates.block_scores(L, ends, block)
        cand = candidates.candidate_blocks(bs, ends, block, n)
        dense = indexer.topk(L, None, ends, k)
        masked = candidates.candidate_mask(L, ends, cand, block)
        for r in range(6):
            np.testing.assert_array_equal(masked[r, : ends[r]], L[r, : ends[r]])
        np.testing.assert_array_equal(indexer.topk(masked, None, ends, k), dense)
        pool = candidates.gather_logits(L, ends, cand, block)
        pe = candidates.gather_row_ends(cand, ends, block, 6)
        np.testing.assert_array_equal(pe, ends)  # the pool is the row itself
        got = candidates.remap_compact_topk(indexer.topk(pool, None, pe, k), cand, block)
        np.testing.assert_array_equal(got, dense)


def test_gather_route_equals_mask_route():
    # two independent routes through the pool select the same positions (ties
    # included: pool slots run in ascending position order) when the pool holds at
    # least k positions: n candidates hold at least (n - 1) * block + 1 of them, the
    # highest one being possibly cut by the row end
    rng = np.random.default_rng(3)
    for ties in (False, True):
        for block, n, k in ((4, 5, 12), (8, 3, 17), (16, 2, 17)):  # k <= (n - 1) * block + 1
            rows, width = 7, 96
            L = rng.integers(-3, 4, (rows, width)).astype(np.float64) if ties else rng.standard_normal((rows, width))
            ends = rng.integers(n * block + block, width + 1, rows)
            bs = candidates.block_scores(L, ends, block)
            cand = candidates.candidate_blocks(bs, ends, block, n)
            assert (cand >= 0).all()
            masked_tk = indexer.topk(candidates.candidate_mask(L, ends, cand, block), None, ends, k)
            pool = candidates.gather_logits(L, ends, cand, block)
            pe = candidates.gather_row_ends(cand, ends, block, rows)
            gather_tk = candidates.remap_compact_topk(indexer.topk(pool, None, pe, k), cand, block)
            np.testing.assert_array_equal(gather_tk, masked_tk)


def test_row_maximum_survives_the_pool():
    # the block holding a row's largest logit has the largest block score, so the
    # two-level top-1 is the dense top-1 for any n >= 1
    rng = np.random.default_rng(4)
    L, ends = _random_step(rng, 9, 80)
    ends = np.maximum(ends, 1)
    for block in (2, 5, 16):
        bs = candidates.block_scores(L, ends, block)
        cand = candidates.candidate_blocks(bs, ends, block, 1)
        pool = candidates.gather_logits(L, ends, cand, block)
        pe = candidates.gather_row_ends(cand, ends, block, 9)
        got = candidates.remap_compact_topk(indexer.topk(pool, None, pe, 1), cand, block)
        np.testing.assert_array_equal(got, indexer.topk(L, None, ends, 1))


def test_row_repeat_shares_a_candidate_row():
    # rows r and r + 1 with row_repeat 2 read candidate row r // 2
    rng = np.random.default_rng(5)
    L, _ = _random_step(rng, 4, 32)
    ends = np.array([32, 30, 20, 17])
    cand = np.array([[0, 3], [1, 2]])
    m = candidates.candidate_mask(L, ends, cand, 8, row_repeat=2)
    for r in range(4):
        keep = [c for c in range(32) if c < ends[r] and c // 8 in cand[r // 2]]
        assert np.isfinite(m[r, keep]).all()
        assert np.isneginf(np.delete(m[r], keep)).all()
    pos = candidates.gather_positions(cand, ends, 8, 4, row_repeat=2)
    assert pos[1, 13] == 29 and pos[1, 15] == -1 and pos[0, 15] == 31 and pos[3, 15] == -1 and pos[3, 8] == 16


def test_remap_keeps_pads():
    cand = np.array([[5, -1]])
    t = np.array([[0, 3, 4, -1, 8, 9]])  # slot 4 has candidate -1; slots 8 and 9 lie past the list
    np.testing.assert_array_equal(candidates.remap_compact_topk(t, cand, 4), [[20, 23, -1, -1, -1, -1]])
