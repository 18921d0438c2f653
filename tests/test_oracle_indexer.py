"""Pins of the oracle's logits, paged cache layout, row ends and top-k.

Each test checks the oracle against something other than itself: hand-worked cases
under tests/golden (each citing the passage it follows), closed forms that reduce to a
library matmul, exact invariants of the formula (sign and scale laws, mask exactness,
permutation of physical pages, paged == contiguous, MTP nesting), and a brute-force
top-k by Python's own sort.
"""

import json
import os

import numpy as np
import pytest
import torch

from oracle import cache, formats, indexer
from sparse_attention_indexer_mxfp4_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f(x):
    return float("-inf") if x == "-inf" else float(x)


# ----------------------------------------------------------------------------------
# hand-worked cases
# ----------------------------------------------------------------------------------
def test_handworked_fp8_contiguous():
    g = _load("handworked_fp8_contiguous.json")
    q = np.zeros((2, 2, 128), np.uint8)
    k = np.zeros((3, 128), np.uint8)
    for e in g["q"]:
        q[e["row"], e["head"], e["lane"]] = int(e["code"], 16)
    for e in g["k"]:
        k[e["key"], e["lane"]] = int(e["code"], 16)
    out = indexer.mqa_logits_fp8(q, k, np.float32(g["k_scale"]), np.float32(g["w"]), g["ks"], g["ke"])
    want = np.array([[_f(v) for v in row] for row in g["expected_logits"]])
    assert np.array_equal(out, want)
    for kk, exp in g["expected_topk"].items():
        assert indexer.topk(out, g["ks"], g["ke"], int(kk)).tolist() == exp


def test_handworked_magnitude():
    # the oracle's magnitude mode (the row scale of the tolerance floor) on a hand-worked
    # input whose dot products cancel, through the contiguous and the paged routes
    g = _load("handworked_magnitude.json")
    q = np.zeros((1, 2, 128), np.uint8)
    k = np.zeros((2, 128), np.uint8)
    for e in g["q"]:
        q[e["row"], e["head"], e["lane"]] = int(e["code"], 16)
    for e in g["k"]:
        k[e["key"], e["lane"]] = int(e["code"], 16)
    ksc, w = np.float32(g["k_scale"]), np.float32(g["w"])
    got = indexer.mqa_logits_fp8(q, k, ksc, w, g["ks"], g["ke"])
    mag = indexer.mqa_logits_fp8(q, k, ksc, w, g["ks"], g["ke"], magnitude=True)
    assert got.tolist() == g["expected_logits"]
    assert mag.tolist() == g["expected_magnitude"]
    P = 16
    pool = np.zeros((1, cache.fp8_page_bytes(P, 128)), np.uint8)
    cache.store_fp8(pool, [0, 1], k, ksc, P)
    pmag = indexer.paged_logits(pool, "fp8", P, np.zeros((1, 1), np.int32), [2], q[None], w, 1, 1, 4,
                                magnitude=True)
    assert pmag[0, :2].tolist() == g["expected_magnitude"][0] and np.isneginf(pmag[0, 2:]).all()


def test_handworked_mxfp4_paged():
    g = _load("handworked_mxfp4_paged.json")
    H, D, P = 2, 128, 64
    qn = np.zeros((1, 1, H, D), np.uint8)
    for e in g["q"]:
        qn[0, 0, e["head"], e["element"]] = int(e["nibble"], 16)
    kn = np.zeros((2, D), np.uint8)
    for e in g["k"]:
        kn[e["key"], e["element"]] = int(e["nibble"], 16)
    q_packed = formats.pack_e2m1(qn)
    q_scale = formats.scales_to_int32(np.array(g["q_scale_bytes"], np.uint8))[None, None, :]
    pool = np.zeros((1, cache.mxfp4_page_bytes(P, D)), np.uint8)
    cache.store_mxfp4(pool, [0, 1], formats.pack_e2m1(kn), np.array(g["k_scale_bytes"], np.uint8), P)
    bt = np.zeros((1, 1), np.int32)
    out = indexer.paged_logits(pool, "mxfp4", P, bt, [g["context_len"]], q_packed, np.float32(g["w"]), 1, 1,
                               g["width"], q_scale=q_scale)
    assert out[0, :3].tolist() == [_f(v) for v in g["expected_logits_first3"]]
    assert np.all(np.isneginf(out[0, 2:]))


def test_page_offsets_golden():
    g = _load("page_offsets.json")
    P, D = 64, 128
    for e in g["fp8"]:
        pool = np.zeros((1, cache.fp8_page_bytes(P, D)), np.uint8)
        codes = np.zeros((1, D), np.uint8)
        scale = np.zeros(1, np.float32)
        if "value_byte" in e:
            codes[0, e["value_byte"]] = 0xAB
        else:
            scale.view(np.uint8)[e["scale_byte"]] = 0xAB
        cache.store_fp8(pool, [e["entry"]], codes, scale, P)
        assert np.flatnonzero(pool[0]).tolist() == [e["offset"]], e
    for e in g["mxfp4"]:
        pool = np.zeros((1, cache.mxfp4_page_bytes(P, D)), np.uint8)
        packed = np.zeros((1, D // 2), np.uint8)
        sb = np.zeros((1, D // 32), np.uint8)
        if "value_byte" in e:
            packed[0, e["value_byte"]] = 0xAB
        else:
            sb[0, e["scale"]] = 0xAB
        cache.store_mxfp4(pool, [e["entry"]], packed, sb, P)
        assert np.flatnonzero(pool[0]).tolist() == [e["offset"]], e


def test_mxfp4_page_is_a_bijection():
    # every byte of the page is written by exactly one (entry, byte) of one store
    P, D = 64, 128
    pool = np.zeros((1, cache.mxfp4_page_bytes(P, D)), np.int64)
    vo, so = cache._mxfp4_offsets(P, D, np.arange(P))
    counts = np.bincount(np.concatenate([vo.ravel(), so.ravel()]), minlength=pool.shape[1])
    assert np.all(counts == 1)
    # a wavefront's 16-byte loads of one run cover one contiguous KiB: lane i of run r,
    # chunk i // 16, entry i % 16 starts at r * 1024 + 16 * i
    for r in range(4):
        for lane in range(64):
            assert vo[16 * r + lane % 16, 16 * (lane // 16)] == r * 1024 + 16 * lane


# ----------------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------------
def _rand_fp8(rng, shape):
    return formats.quant_e4m3(rng.standard_normal(shape).astype(np.float32) * 4)


def test_one_hot_weights_reduce_to_matmul():
    rng = np.random.default_rng(20)
    M, N, H, D = 5, 37, 3, 128
    q = _rand_fp8(rng, (M, H, D))
    k = _rand_fp8(rng, (N, D))
    ks = np.float32(rng.uniform(0.01, 2, N))
    for h0 in range(H):
        w = np.zeros((M, H), np.float32)
        w[:, h0] = 1.0
        out = indexer.mqa_logits_fp8(q, k, ks, w, np.zeros(M), np.full(M, N))
        qt = torch.from_numpy(formats.decode_e4m3(q[:, h0, :]))
        kt = torch.from_numpy(formats.decode_e4m3(k))
        ref = torch.relu(torch.matmul(qt, kt.T) * torch.from_numpy(ks.astype(np.float64))[None, :]).numpy()
        np.testing.assert_allclose(out, ref, rtol=1e-15, atol=0)


def test_single_head_nonnegative_is_plain_matmul():
    rng = np.random.default_rng(21)
    M, N, D = 7, 29, 128
    q = formats.quant_e4m3(np.abs(rng.standard_normal((M, 1, D))).astype(np.float32))
    k = formats.quant_e4m3(np.abs(rng.standard_normal((N, D))).astype(np.float32))
    out = indexer.mqa_logits_fp8(q, k, np.ones(N, np.float32), np.ones((M, 1), np.float32),
                                 np.zeros(M), np.full(M, N))
    ref = torch.matmul(torch.from_numpy(formats.decode_e4m3(q[:, 0])), torch.from_numpy(formats.decode_e4m3(k)).T)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-15, atol=0)


# ----------------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------------
def _contig_case(seed, M=6, N=50, H=4):
    rng = np.random.default_rng(seed)
    q = _rand_fp8(rng, (M, H, 128))
    k = _rand_fp8(rng, (N, 128))
    ks = np.float32(rng.uniform(0.01, 2, N))
    w = rng.standard_normal((M, H)).astype(np.float32)
    starts = rng.integers(0, N // 2, M)
    ends = rng.integers(N // 2, N + 1, M)
    return q, k, ks, w, starts, ends


def test_mask_exactness():
    q, k, ks, w, st, en = _contig_case(30)
    out = indexer.mqa_logits_fp8(q, k, ks, w, st, en)
    cols = np.arange(out.shape[1])
    valid = (cols[None] >= st[:, None]) & (cols[None] < en[:, None])
    assert np.array_equal(np.isfinite(out), valid)
    assert np.all(np.isneginf(out[~valid]))


def test_weight_sign_and_scale_laws():
    q, k, ks, w, st, en = _contig_case(31)
    base = indexer.mqa_logits_fp8(q, k, ks, w, st, en)
    fin = np.isfinite(base)
    neg = indexer.mqa_logits_fp8(q, k, ks, -w, st, en)
    assert np.array_equal(neg[fin], -base[fin])
    dbl = indexer.mqa_logits_fp8(q, k, ks, 2 * w, st, en)
    assert np.array_equal(dbl[fin], 2 * base[fin])
    dks = indexer.mqa_logits_fp8(q, k, 2 * ks, w, st, en)
    assert np.array_equal(dks[fin], 2 * base[fin])


def test_relu_is_per_head():
    # a head whose scores are all negative contributes nothing, whatever its weight
    rng = np.random.default_rng(32)
    M, N = 3, 20
    q = np.zeros((M, 2, 128), np.uint8)
    q[:, 0, 0] = formats.quant_e4m3(np.float32([1.0]))[0]
    q[:, 1, 0] = formats.quant_e4m3(np.float32([-1.0]))[0]
    k = np.zeros((N, 128), np.uint8)
    k[:, 0] = formats.quant_e4m3(np.abs(rng.standard_normal(N)).astype(np.float32) + 0.1)
    w = np.float32([[1.0, 5.0]] * M)
    out = indexer.mqa_logits_fp8(q, k, np.ones(N, np.float32), w, np.zeros(M), np.full(M, N))
    np.testing.assert_array_equal(out, np.tile(formats.decode_e4m3(k[:, 0])[None], (M, 1)))


def _paged_case(seed, fmt, B=3, next_n=2, H=4, lens=(70, 1, 200), width=256, stride_pad=0):
    wl = workloads.paged(seed, B=B, next_n=next_n, H=H, ctx_lo=0, ctx_hi=0, width=width, topk=8, fmt=fmt,
                         context_lens=np.array(lens))
    P, D = wl.page_size, wl.D
    if fmt == "fp8":
        pb = cache.fp8_page_bytes(P, D)
        pool = np.zeros((wl.num_pages, pb + stride_pad), np.uint8)
        codes, sc = formats.quantize_k_fp8(wl.k)
        cache.store_fp8(pool, wl.slot_mapping, codes, sc, P)
        q = formats.quantize_fp8_noscale(wl.q)
        qs = None
    else:
        pb = cache.mxfp4_page_bytes(P, D)
        pool = np.zeros((wl.num_pages, pb + stride_pad), np.uint8)
        packed, sb = formats.quantize_mxfp4(wl.k)
        cache.store_mxfp4(pool, wl.slot_mapping, packed, sb, P)
        q, qsb = formats.quantize_mxfp4(wl.q)
        qs = formats.scales_to_int32(qsb)
    return wl, pool, q, qs


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_paged_equals_contiguous(fmt):
    wl, pool, q, qs = _paged_case(33, fmt)
    out = indexer.paged_logits(pool, fmt, wl.page_size, wl.block_table, wl.context_lens, q, wl.w,
                               wl.B, wl.next_n, wl.width, q_scale=qs)
    ends = indexer.paged_row_ends(wl.context_lens, wl.B, wl.next_n)
    for b in range(wl.B):
        L = int(wl.context_lens[b])
        kk = wl.k[wl.key_offsets[b]: wl.key_offsets[b] + L]
        rows = slice(b * wl.next_n, (b + 1) * wl.next_n)
        if fmt == "fp8":
            codes, sc = formats.quantize_k_fp8(kk)
            ref = indexer.logits_from_values(formats.decode_e4m3(q[b]), formats.decode_e4m3(codes), wl.w[rows],
                                             np.zeros(wl.next_n), ends[rows], k_scale=sc, width=wl.width)
        else:
            packed, sb = formats.quantize_mxfp4(kk)
            qv = formats.decode_mxfp4(q[b], formats.scales_from_int32(qs[b]))
            ref = indexer.logits_from_values(qv, formats.decode_mxfp4(packed, sb), wl.w[rows],
                                             np.zeros(wl.next_n), ends[rows], width=wl.width)
        assert np.array_equal(out[rows], ref)


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_page_permutation_invariance(fmt):
    wl, pool, q, qs = _paged_case(34, fmt, stride_pad=32)
    out = indexer.paged_logits(pool, fmt, wl.page_size, wl.block_table, wl.context_lens, q, wl.w,
                               wl.B, wl.next_n, wl.width, q_scale=qs)
    perm = np.random.default_rng(1).permutation(wl.num_pages)
    pool2 = np.empty_like(pool)
    pool2[perm] = pool
    bt2 = perm[wl.block_table]
    out2 = indexer.paged_logits(pool2, fmt, wl.page_size, bt2, wl.context_lens, q, wl.w,
                                wl.B, wl.next_n, wl.width, q_scale=qs)
    assert np.array_equal(out, out2)


def test_mtp_rows_are_nested():
    wl, pool, q, qs = _paged_case(35, "fp8", next_n=3, lens=(130, 64, 2))
    out = indexer.paged_logits(pool, "fp8", wl.page_size, wl.block_table, wl.context_lens, q, wl.w,
                               wl.B, wl.next_n, wl.width)
    fin = np.isfinite(out).reshape(wl.B, wl.next_n, -1)
    for b in range(wl.B):
        L = int(wl.context_lens[b])
        for j in range(wl.next_n):
            assert fin[b, j].sum() == max(L - wl.next_n + j + 1, 0)
            assert np.array_equal(np.flatnonzero(fin[b, j]), np.arange(max(L - wl.next_n + j + 1, 0)))


def test_per_row_lengths_match_per_sequence():
    wl, pool, q, qs = _paged_case(36, "fp8", next_n=2, lens=(90, 5, 64))
    a = indexer.paged_logits(pool, "fp8", wl.page_size, wl.block_table, wl.context_lens, q, wl.w,
                             wl.B, wl.next_n, wl.width)
    per_row = indexer.paged_row_ends(wl.context_lens, wl.B, wl.next_n)
    b = indexer.paged_logits(pool, "fp8", wl.page_size, wl.block_table, per_row, q, wl.w,
                             wl.B, wl.next_n, wl.width, per_row=True)
    assert np.array_equal(a, b)


def test_mxfp4_unit_scales_match_plain_e2m1():
    rng = np.random.default_rng(37)
    qn = rng.integers(0, 16, (1, 1, 2, 128)).astype(np.uint8)
    kn = rng.integers(0, 16, (10, 128)).astype(np.uint8)
    P, D = 64, 128
    pool = np.zeros((1, cache.mxfp4_page_bytes(P, D)), np.uint8)
    cache.store_mxfp4(pool, np.arange(10), formats.pack_e2m1(kn), np.full((10, 4), 127, np.uint8), P)
    qs = formats.scales_to_int32(np.full((1, 1, 2, 4), 127, np.uint8))
    w = np.float32([[0.3, -1.2]])
    out = indexer.paged_logits(pool, "mxfp4", P, np.zeros((1, 1), np.int32), [10], formats.pack_e2m1(qn), w,
                               1, 1, 64, q_scale=qs)
    qv = formats.decode_e2m1(qn[0, 0])
    kv = formats.decode_e2m1(kn)
    ref = sum(float(w[0, h]) * np.maximum(qv[h] @ kv.T, 0) for h in range(2))
    np.testing.assert_allclose(out[0, :10], ref, rtol=1e-15, atol=0)
    # raising one block's key scale by one doubles exactly that block's share
    kn2 = np.zeros((1, 128), np.uint8)
    kn2[0, 40] = 0x2  # 1.0 in block 1
    qn2 = np.zeros((1, 1, 1, 128), np.uint8)
    qn2[..., 40] = 0x4  # 2.0
    for e in (127, 128, 131):
        pool = np.zeros((1, cache.mxfp4_page_bytes(P, D)), np.uint8)
        cache.store_mxfp4(pool, [0], formats.pack_e2m1(kn2), np.array([[127, e, 127, 127]], np.uint8), P)
        o = indexer.paged_logits(pool, "mxfp4", P, np.zeros((1, 1), np.int32), [1], formats.pack_e2m1(qn2),
                                 np.float32([[1.0]]), 1, 1, 64,
                                 q_scale=formats.scales_to_int32(np.full((1, 1, 1, 4), 127, np.uint8)))
        assert o[0, 0] == 2.0 * 2.0 ** (e - 127)


def test_row_ends_rule():
    ends = indexer.paged_row_ends([10, 1, 0], 3, 2)
    assert ends.tolist() == [9, 10, 0, 1, 0, 0]


# ----------------------------------------------------------------------------------
# top-k
# ----------------------------------------------------------------------------------
def _topk_brute(row, start, end, k):
    items = sorted(((-row[c], c) for c in range(start, end)))
    chosen = sorted(c for _, c in items[:k])
    return [c - start for c in chosen] + [-1] * (k - len(chosen))


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(40)
    R, W = 60, 90
    vals = rng.integers(-4, 5, (R, W)).astype(np.float64)  # many ties
    vals[rng.random((R, W)) < 0.1] = -np.inf
    starts = rng.integers(0, 40, R)
    ends = rng.integers(0, W + 1, R)
    for k in (1, 5, 17, 64, 100):
        got = indexer.topk(vals, starts, ends, k)
        for r in range(R):
            assert got[r].tolist() == _topk_brute(vals[r].tolist(), int(starts[r]), max(int(ends[r]), int(starts[r])), k)


def test_topk_selected_dominate_unselected():
    rng = np.random.default_rng(41)
    L = rng.standard_normal((20, 500))
    got = indexer.topk(L, None, np.full(20, 500), 37)
    for r in range(20):
        sel = np.zeros(500, bool)
        sel[got[r]] = True
        assert L[r, sel].min() >= L[r, ~sel].max()


def test_topk_signed_zero_ties():
    row = np.array([[0.0, -0.0, 0.0, -1.0]])
    assert indexer.topk(row, [0], [4], 2).tolist() == [[0, 1]]


def test_topk_to_slots_handworked():
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "handworked_topk_slots.json")))
    slots, indptr, lens = indexer.topk_to_slots(np.array(g["topk"]), g["row_seq"], np.array(g["block_table"]),
                                                g["page_size"], g["row_valid"])
    np.testing.assert_array_equal(slots, g["slots"])
    np.testing.assert_array_equal(indptr, g["indptr"])
    np.testing.assert_array_equal(lens, g["lens"])


def test_topk_to_slots_inverts_the_page_layout():
    # a slot names a page entry; reading the block table backwards recovers the
    # local position from each slot
    rng = np.random.default_rng(11)
    P, B, mb = 16, 3, 8
    perm = rng.permutation(B * mb)
    bt = perm.reshape(B, mb)
    topk = rng.integers(-1, P * mb, (6, 10))
    seq = np.array([0, 0, 1, 1, 2, 2])
    slots, indptr, lens = indexer.topk_to_slots(topk, seq, bt, P)
    inv = {int(page): (b, blk) for b in range(B) for blk, page in enumerate(bt[b])}
    for r in range(6):
        kept = topk[r][topk[r] >= 0]
        got = slots[indptr[r]:indptr[r + 1]]
        assert len(got) == len(kept) == lens[r]
        for s, p in zip(got, kept):
            b, blk = inv[int(s) // P]
            assert b == seq[r] and blk * P + int(s) % P == p
