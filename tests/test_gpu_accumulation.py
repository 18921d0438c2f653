"""The matrix cores' accumulation error on adversarial dot products, measured through
the C ABI and asserted, since the tolerance floor of the parity tests rests on it.

Two heads with q[t, 1, :] = -q[t, 0, :], weights (1, -1) and unit key scales make the
logit the raw dot product: ReLU(S) - ReLU(-S) = S exactly, and the kernels' head sums
add a zero. So |I_gpu - I_oracle| is the error of one 128-term fp8 (or scaled fp4)
dot product, and the oracle's magnitude A = 2 * sum_d |q_d k_d| gives its scale.

The operands are built to stress an accumulator that aligns products before adding
them: one product of the largest e4m3 size beside many far smaller ones (their low
bits fall below the big one's alignment), two such products cancelling, uniformly
random codes over the whole finite range, and 32-channel groups of very different
exponents. MXFP4 keys get block scales up to 2^20 apart.

Measured on an MI355X: the fp8 worst case is 2^-11.98 of sum_d |q_d k_d| (as if each
of the 128 products were cut to 19 bits below the largest: 128 * 2^-19 = 2^-12), the
scaled fp4 one far smaller. The bound asserted, 2^-11.75, stays below the floor the
parity tests use for degenerate rows (2^-11 of the same size) by a factor 1.2, and
the measured worst ratio is printed.
"""

import numpy as np
import pytest
import torch

from oracle import cache, formats, indexer
from sparse_attention_indexer_mxfp4_amd import ops

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
D = 128
ROWS = 8
KEYS = 4096
P = 64
BOUND = 2.0 ** -11.75


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _e4m3(sign, e, m):
    """e4m3fn codes from fields (e in 0..15, m in 0..7; e = 15 with m = 7 is NaN, avoided)."""
    m = np.where((e == 15) & (m == 7), 6, m)
    return ((sign.astype(np.int64) << 7) | (e.astype(np.int64) << 3) | m).astype(np.uint8)


def _fp8_operands(rng):
    def rnd(shape, elo, ehi):
        return _e4m3(rng.integers(0, 2, shape), rng.integers(elo, ehi + 1, shape), rng.integers(0, 8, shape))

    q = np.empty((ROWS, D), np.uint8)
    q[0] = 0x7E  # 448 everywhere
    q[1] = 0x38  # 1.0 everywhere
    # no query spans more than 13 binades: the prefill kernels carry sum_h w_h q_h as
    # e4m3 parts of a row-scaled copy, exact only while its smallest entries stay
    # normal, and this test measures the matrix cores, not that split
    q[2] = rnd(D, 2, 15)
    q[3] = rnd(D, 12, 15)
    for r in range(4, ROWS):
        q[r] = rnd(D, 1, 14)
    k = np.empty((KEYS, D), np.uint8)
    kind = np.arange(KEYS) % 4
    for s in range(KEYS):
        if kind[s] in (0, 1):
            k[s] = rnd(D, 1, 8)  # far below the big product's size
            k[s, rng.integers(0, D)] = 0x7E
            if kind[s] == 1:  # a big pair that cancels
                k[s, (rng.integers(1, D) + np.flatnonzero(k[s] == 0x7E)[0]) % D] = 0xFE
        elif kind[s] == 2:
            k[s] = rnd(D, 0, 15)
        else:
            base = rng.integers(1, 15, 4)
            e = np.clip(np.repeat(base, 32) + rng.integers(-1, 2, D), 0, 15)
            k[s] = _e4m3(rng.integers(0, 2, D), e, rng.integers(0, 8, D))
    return q, k


def _ratio(got, exact, mag):
    fin = np.isfinite(exact)
    assert np.array_equal(np.isfinite(got), fin)
    scale = mag[fin] / 2.0  # sum_d |q_d k_d|
    nz = scale > 0
    err = np.abs(got[fin] - exact[fin])
    assert np.all(err[~nz] == 0.0)
    return float((err[nz] / scale[nz]).max())


def test_fp8_accumulation_bound():
    rng = np.random.default_rng(2024)
    q, k = _fp8_operands(rng)
    q2 = np.stack([q, q ^ np.uint8(0x80)], axis=1)  # [ROWS, 2, D]: the second head negated
    w = np.tile(np.float32([1.0, -1.0]), (ROWS, 1))
    ones = np.ones(KEYS, np.float32)
    ks, ke = np.zeros(ROWS, np.int32), np.full(ROWS, KEYS, np.int32)
    exact = indexer.mqa_logits_fp8(q2, k, ones, w, ks, ke)
    mag = indexer.mqa_logits_fp8(q2, k, ones, w, ks, ke, magnitude=True)

    # decode walk over a paged cache (every row its own sequence over the same pages)
    pool = np.zeros((KEYS // P, cache.fp8_page_bytes(P, D)), np.uint8)
    cache.store_fp8(pool, np.arange(KEYS), k, ones, P)
    bt = np.tile(np.arange(KEYS // P, dtype=np.int32), (ROWS, 1))
    dec, _ = ops.idx_paged_mqa_logits(_dev(pool), ops.FP8, P, _dev(q2[:, None]), None, _dev(w),
                                      _dev(np.full(ROWS, KEYS, np.int32)), _dev(bt), KEYS)
    # prefill kernel (its |x| split carries the linear term on one more MFMA)
    pre = ops.idx_mqa_logits(_dev(q2), _dev(k), _dev(ones), _dev(w), _dev(ks), _dev(ke))
    # MTP walk, two rows per sequence and 64 heads (62 of them zero): the kernel of the
    # multi-row decode steps
    H2, B2 = 64, ROWS // 2
    q64 = np.zeros((ROWS, H2, D), np.uint8)
    q64[:, :2] = q2
    w64 = np.zeros((ROWS, H2), np.float32)
    w64[:, :2] = w
    lens2 = np.full(B2, KEYS, np.int32)
    bt2 = np.tile(np.arange(KEYS // P, dtype=np.int32), (B2, 1))
    mtp_args = (pool, "fp8", P, bt2, lens2, q64.reshape(B2, 2, H2, D), w64, B2, 2, KEYS)
    mtp_exact = indexer.paged_logits(*mtp_args)
    mtp_mag = indexer.paged_logits(*mtp_args, magnitude=True)
    mtp, _ = ops.idx_paged_mqa_logits(_dev(pool), ops.FP8, P, _dev(q64.reshape(B2, 2, H2, D)), None, _dev(w64),
                                      _dev(lens2), _dev(bt2), KEYS)
    torch.cuda.synchronize()
    r_dec = _ratio(dec.cpu().numpy().astype(np.float64), exact, mag)
    r_pre = _ratio(pre.cpu().numpy().astype(np.float64), exact, mag)
    r_mtp = _ratio(mtp.cpu().numpy().astype(np.float64), mtp_exact, mtp_mag)
    print(f"fp8 worst |err| / sum|q k|: decode walk 2^{np.log2(max(r_dec, 1e-300)):.2f}, "
          f"prefill 2^{np.log2(max(r_pre, 1e-300)):.2f}, MTP walk 2^{np.log2(max(r_mtp, 1e-300)):.2f}", flush=True)
    assert r_dec <= BOUND
    assert r_pre <= BOUND
    assert r_mtp <= BOUND


def test_mxfp4_accumulation_bound():
    rng = np.random.default_rng(2025)
    qn = rng.integers(0, 16, (ROWS, D)).astype(np.uint8)
    qn[0] = 0x7  # 6.0 everywhere
    kn = rng.integers(0, 16, (KEYS, D)).astype(np.uint8)
    kind = np.arange(KEYS) % 4
    kn[kind == 0, 0] = 0x7
    ksb = np.full((KEYS, D // 32), 127, np.uint8)
    for s in range(KEYS):
        if kind[s] == 0:
            ksb[s] = [147, *rng.integers(120, 131, 3)]  # one block 2^20 above the rest
        elif kind[s] == 1:
            ksb[s] = rng.integers(107, 148, 4)
        elif kind[s] == 2:
            ksb[s] = 127 + rng.integers(-2, 3, 4)
        else:
            ksb[s] = [137, 137, *rng.integers(117, 121, 2)]
            kn[s, 32:64] = kn[s, 0:32] ^ 0x8  # block 0 negated (cancels it for row 0)
    # query block scales within 2^4 of each other (the prefill kernels' exact range for
    # sum_h w_h q_h, as above); row 0 uniform
    qsb = rng.integers(125, 130, (ROWS, D // 32)).astype(np.uint8)
    qsb[0] = 127
    qp = formats.pack_e2m1(np.stack([qn, qn ^ 0x8], axis=1))  # [ROWS, 2, 64]
    qs = formats.scales_to_int32(np.stack([qsb, qsb], axis=1))  # [ROWS, 2]
    w = np.tile(np.float32([1.0, -1.0]), (ROWS, 1))
    pool = np.zeros((KEYS // P, cache.mxfp4_page_bytes(P, D)), np.uint8)
    cache.store_mxfp4(pool, np.arange(KEYS), formats.pack_e2m1(kn), ksb, P)
    bt = np.tile(np.arange(KEYS // P, dtype=np.int32), (ROWS, 1))
    lens = np.full(ROWS, KEYS, np.int32)
    args = (pool, "mxfp4", P, bt, lens, qp[:, None], w, ROWS, 1, KEYS)
    exact = indexer.paged_logits(*args, q_scale=qs[:, None])
    mag = indexer.paged_logits(*args, q_scale=qs[:, None], magnitude=True)
    dec, _ = ops.idx_paged_mqa_logits(_dev(pool), ops.MXFP4, P, _dev(qp[:, None]), _dev(qs[:, None]), _dev(w),
                                      _dev(lens), _dev(bt), KEYS)
    # the prefill chunk kernel over the same pages (rows of one sequence)
    pre = ops.idx_paged_prefill_logits(_dev(pool), ops.MXFP4, P, _dev(qp), _dev(qs), _dev(w), _dev(lens),
                                       _dev(bt[0]), KEYS)
    torch.cuda.synchronize()
    r_dec = _ratio(dec.cpu().numpy().astype(np.float64), exact, mag)
    r_pre = _ratio(pre.cpu().numpy().astype(np.float64), exact, mag)
    print(f"MXFP4 worst |err| / sum|q k|: decode walk 2^{np.log2(max(r_dec, 1e-300)):.2f}, "
          f"prefill chunk 2^{np.log2(max(r_pre, 1e-300)):.2f}", flush=True)
    assert r_dec <= BOUND
    assert r_pre <= BOUND
