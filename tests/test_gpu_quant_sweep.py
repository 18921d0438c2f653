"""Every-pattern parity of the quantisers with the oracle (byte work: bit for bit).

How fp32 rounds to e4m3 or e2m1 depends only on the value's bits, so these tests put
whole ranges of bit patterns through the kernels and compare every output byte with
the oracle's:

* fp8 query (e4m3 of the value itself): every fp32 bit pattern. In the 19 binades
  [2^-10, 2^9), where the code changes, every one of the 2^23 mantissas goes through
  the kernel and the oracle. In every other binade the oracle gives one code at both
  ends; rounding to nearest is monotone in |x|, so that code is the oracle's answer
  for the whole binade, and all 2^23 kernel outputs are compared with it. NaN
  patterns give the NaN code (the oracle has no answer for NaN: the kernel's own
  documented behaviour is checked instead).
* MXFP4 query: blocks of 32 whose first value fixes the block's e8m0 byte at 127, 0
  or 253 (amax 6, 6 * 2^-127 and the largest finite fp32). The other 31 values run
  over every pattern whose scaled magnitude is in [2^-3, 6] (e2m1 codes change in
  [0.25, 6]), plus sampled mantissas of every binade below. A further set of blocks
  takes as amax every binade at the mantissas where the e8m0 rule turns.
* K store, fp8 and MXFP4: rows whose amax fixes the scale (448: quotients exact;
  1000: quotients rounded; 2^-120: a subnormal fp32 scale), the other values of the
  row running over every pattern of chosen binades.
* bf16 inputs: every bf16 pattern, for both query formats.

Negative inputs: the oracle's codes are sign-magnitude, so the code of -x is that of
x with the sign bit flipped. Each sweep checks this on a sample of negated inputs
through the oracle itself, then compares the kernel on every negated input with the
codes of the positive ones, sign bits flipped.
"""

import numpy as np
import pytest
import torch

from oracle import cache, formats
from sparse_attention_indexer_mxfp4_amd import ops

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
MANT = 1 << 23
ROWS = 1 << 16  # rows of 128 values per kernel call in the binade sweeps


def _bits_range(lo: int, hi: int) -> np.ndarray:
    """fp32 values whose bit patterns are lo .. hi (inclusive, same sign)."""
    return np.arange(lo, hi + 1, dtype=np.uint64).astype(np.uint32).view(np.float32)


def _binade_bits(e_biased: int, sign: int = 0) -> int:
    return (sign << 31) | (e_biased << 23)


def _gpu_patterns(hi_bits: int) -> torch.Tensor:
    """On the device: the 2^23 fp32 values hi_bits | m, m = 0 .. 2^23 - 1, as [2^16, 1, 128]."""
    hi = int(np.array([hi_bits], dtype=np.uint32).view(np.int32)[0])
    return (torch.arange(MANT, dtype=torch.int32, device=DEV) | hi).view(torch.float32).view(ROWS, 1, 128)


def _first_diff(got: np.ndarray, want: np.ndarray, inputs: np.ndarray | None = None) -> str:
    """The mismatch count and the first few (flat index, got, want[, input])."""
    got, want = got.reshape(-1), want.reshape(-1)
    bad = np.flatnonzero(got != want)
    i = bad[:5]
    msg = f"{bad.size} mismatches; at {i.tolist()}: got {got[i].tolist()}, want {want[i].tolist()}"
    if inputs is not None:
        msg += f", inputs {inputs.reshape(-1)[i].tolist()}"
    return msg


def _sign_rule_holds(values: np.ndarray, codes: np.ndarray, quant, sign_bits: int, step: int = 97):
    """The oracle gives a sample of the negated rows the same codes with the sign bits flipped."""
    sample = np.ascontiguousarray(values.reshape(-1, values.shape[-1])[::step])
    want = codes.reshape(-1, codes.shape[-1])[::step] ^ np.uint8(sign_bits)
    np.testing.assert_array_equal(quant(-sample), want)


# ----------------------------------------------------------------------------------
# fp8 query: every fp32 pattern
# ----------------------------------------------------------------------------------
FP8_WINDOW = range(127 - 10, 127 + 9)  # biased exponents of [2^-10, 2^9)


def test_q_fp8_every_fp32_pattern():
    for e in range(256):
        pos_gpu = _gpu_patterns(_binade_bits(e))
        neg_gpu = _gpu_patterns(_binade_bits(e, 1))
        if e == 255:
            # +-inf saturate like any magnitude past 448; every other pattern is NaN
            inf = np.array([np.inf, -np.inf], dtype=np.float32)
            want_inf = formats.quantize_fp8_noscale(inf)
            for g, w in ((pos_gpu, want_inf[0]), (neg_gpu, want_inf[1])):
                got = ops.idx_q_quant(g, ops.FP8)[0].view(-1)
                assert int(got[0]) == int(w)
                nan_code = 0x7F | (int(w) & 0x80)
                assert bool((got[1:] == nan_code).all()), "NaN patterns must give the NaN code"
            continue
        got_pos = ops.idx_q_quant(pos_gpu, ops.FP8)[0].view(-1)
        got_neg = ops.idx_q_quant(neg_gpu, ops.FP8)[0].view(-1)
        if e in FP8_WINDOW:
            vals = _bits_range(_binade_bits(e), _binade_bits(e) + MANT - 1)
            want = formats.quantize_fp8_noscale(vals)
            _sign_rule_holds(vals.reshape(-1, 128), want.reshape(-1, 128), formats.quantize_fp8_noscale, 0x80)
            w = torch.from_numpy(want).to(DEV)
            if not torch.equal(got_pos, w):
                pytest.fail(f"binade {e}, +: " + _first_diff(got_pos.cpu().numpy(), want, vals))
            if not torch.equal(got_neg, w ^ 0x80):
                pytest.fail(f"binade {e}, -: " + _first_diff(got_neg.cpu().numpy(), want ^ 0x80, -vals))
        else:
            ends = np.array([_binade_bits(e), _binade_bits(e) + MANT - 1], dtype=np.uint32).view(np.float32)
            want = formats.quantize_fp8_noscale(np.concatenate([ends, -ends]))
            assert want[0] == want[1] and want[2] == want[3], f"binade {e} is not constant in the oracle"
            assert bool((got_pos == int(want[0])).all()), f"binade {e}, +: expected code {int(want[0]):#x} throughout"
            assert bool((got_neg == int(want[2])).all()), f"binade {e}, -: expected code {int(want[2]):#x} throughout"


# ----------------------------------------------------------------------------------
# MXFP4 query: anchored blocks
# ----------------------------------------------------------------------------------
def _f32(bits: int) -> np.float32:
    return np.array([bits], dtype=np.uint32).view(np.float32)[0]


# (e8m0 byte, the block's amax, bit range of the swept values: scaled magnitude [2^-3, 6])
MX_ANCHORS = [
    (127, _f32(0x40C00000), 0x3E000000, 0x40C00000),  # amax 6: scale 1
    (0, _f32(0x01400000), 0x00080000, 0x01400000),  # amax 6 * 2^-127: subnormal inputs, scale 2^127
    (253, _f32(0x7F7FFFFF), 0x7D000000, 0x7F7FFFFF),  # largest finite amax: scale 2^-126
]


def _anchor_rows(anchor: np.float32, vals: np.ndarray, per: int, row: int) -> np.ndarray:
    """Groups of `per` values: the anchor then per-1 of `vals` (zero-padded), as rows of `row`."""
    body = per - 1
    n = -(-vals.size // body)
    n = -(-n // (row // per)) * (row // per)
    b = np.zeros(n * body, np.float32)
    b[:vals.size] = vals
    g = np.concatenate([np.full((n, 1), anchor, np.float32), b.reshape(n, body)], axis=1)
    return g.reshape(-1, row)


def _below_window_samples(lo_bits: int, rng) -> np.ndarray:
    """Sampled mantissas of every binade below lo_bits (subnormals included)."""
    out = []
    for e in range(0, (lo_bits >> 23) + 1):
        m = np.concatenate([[0, 1, 0x3FFFFF, 0x400000, 0x400001, 0x7FFFFF], rng.integers(0, MANT, 26)])
        b = (e << 23) | m.astype(np.uint32)
        out.append(b[b < lo_bits])
    return np.concatenate(out).astype(np.uint32).view(np.float32)


def _check_mx_rows(rows: np.ndarray, tag: str):
    q = torch.from_numpy(rows).to(DEV).view(rows.shape[0], 1, 128)
    packed, sb = formats.quantize_mxfp4(rows)
    want_s = formats.scales_to_int32(sb)
    _sign_rule_holds(rows, packed, lambda x: formats.quantize_mxfp4(x)[0], 0x88)
    for sgn, q_in, wp in ((1, q, packed), (-1, -q, packed ^ np.uint8(0x88))):
        out, sc = ops.idx_q_quant(q_in, ops.MXFP4)
        got = out.view(rows.shape[0], 64).cpu().numpy()
        if not np.array_equal(got, wp):
            pytest.fail(f"{tag} sign {sgn} (packed bytes, two inputs each): " + _first_diff(got, wp))
        np.testing.assert_array_equal(sc.view(-1).cpu().numpy(), want_s, err_msg=f"{tag} sign {sgn}: e8m0 bytes")


@pytest.mark.parametrize("bits,anchor,lo,hi", MX_ANCHORS, ids=[f"e8m0_{a[0]}" for a in MX_ANCHORS])
def test_q_mxfp4_every_pattern_at_scale(bits, anchor, lo, hi):
    assert formats.e8m0_block_bits(np.float64(anchor)) == bits
    rng = np.random.default_rng(200 + bits)
    chunk = 31 * 4 * ROWS
    for c0 in range(lo, hi + 1, chunk):
        vals = _bits_range(c0, min(hi, c0 + chunk - 1))
        _check_mx_rows(_anchor_rows(anchor, vals, 32, 128), f"amax {anchor!r}, bits {c0:#x}..")
    below = _below_window_samples(lo, rng)
    _check_mx_rows(_anchor_rows(anchor, below, 32, 128), f"amax {anchor!r}, below the window")


def test_q_mxfp4_every_amax_binade():
    # one block per amax: every binade at the mantissas where the e8m0 rule turns
    # (f = 1.5 is the boundary), the rest of the block below the amax
    rng = np.random.default_rng(210)
    m = np.array([0, 1, 0x200000, 0x3FFFFF, 0x400000, 0x400001, 0x7FFFFE, 0x7FFFFF], dtype=np.uint32)
    m = np.concatenate([m, rng.integers(0, MANT, 8).astype(np.uint32)])
    amax = ((np.arange(255, dtype=np.uint32)[:, None] << 23) | m[None, :]).reshape(-1).view(np.float32)
    frac = rng.random((amax.size, 31)).astype(np.float32)
    frac[:, :4] = [1.0, 0.5, 0.25, 0.0]
    body = (amax[:, None] * frac).astype(np.float32)
    body *= np.where(rng.random(body.shape) < 0.5, np.float32(-1), np.float32(1))
    blocks = np.concatenate([amax[:, None], body], axis=1)
    pad = (-blocks.shape[0]) % 4
    blocks = np.concatenate([blocks, np.zeros((pad, 32), np.float32)])
    _check_mx_rows(blocks.reshape(-1, 128), "amax sweep")


# ----------------------------------------------------------------------------------
# K store
# ----------------------------------------------------------------------------------
def _k_store(rows: np.ndarray, fmt: int, P: int = 64):
    N = rows.shape[0]
    pages = -(-N // P)
    pb = (cache.fp8_page_bytes if fmt == ops.FP8 else cache.mxfp4_page_bytes)(P, 128)
    pool = torch.zeros((pages, pb), dtype=torch.uint8, device=DEV)
    slots = torch.arange(N, dtype=torch.int64, device=DEV)
    ops.idx_k_store(pool, fmt, P, torch.from_numpy(rows).to(DEV), slots)
    return pool.cpu().numpy(), np.arange(N)


# (amax, bit ranges swept): amax 448 gives scale 1; 1000 a rounded scale; 2^-120 a
# subnormal scale (2^-120 / 448)
K_FP8_CASES = [
    (np.float32(448.0), [(0x3A800000, 0x3AFFFFFF), (0x43800000, 0x43E00000)]),
    (np.float32(1000.0), [(0x3B000000, 0x3B7FFFFF), (0x3F800000, 0x3FFFFFFF), (0x44000000, 0x447A0000)]),
    (_f32(0x03800000), [(0x03000000, 0x037FFFFF), (0x00200000, 0x003FFFFF)]),
]


@pytest.mark.parametrize("anchor,ranges", K_FP8_CASES, ids=["amax448", "amax1000", "amax2^-120"])
def test_k_store_fp8_every_pattern(anchor, ranges):
    chunk = 127 * ROWS
    for lo, hi in ranges:
        for c0 in range(lo, hi + 1, chunk):
            rows = _anchor_rows(anchor, _bits_range(c0, min(hi, c0 + chunk - 1)), 128, 128)
            codes, sc = formats.quantize_k_fp8(rows)
            _sign_rule_holds(rows, codes, lambda x: formats.quantize_k_fp8(x)[0], 0x80)
            for sgn in (1, -1):
                pool, slots = _k_store(rows * np.float32(sgn), ops.FP8)
                got, got_sc = cache.load_fp8(pool, slots, 64, 128)
                want = codes if sgn > 0 else codes ^ np.uint8(0x80)
                if not np.array_equal(got, want):
                    pytest.fail(f"amax {anchor!r} bits {c0:#x}.. sign {sgn}: " + _first_diff(got, want, rows * sgn))
                np.testing.assert_array_equal(got_sc.view(np.uint32), sc.view(np.uint32))


def test_k_store_mxfp4_every_pattern():
    bits, anchor, lo, hi = MX_ANCHORS[0]
    chunk = 31 * 4 * ROWS
    for c0 in range(lo, hi + 1, chunk):
        rows = _anchor_rows(anchor, _bits_range(c0, min(hi, c0 + chunk - 1)), 32, 128)
        packed, sb = formats.quantize_mxfp4(rows)
        for sgn in (1, -1):
            pool, slots = _k_store(rows * np.float32(sgn), ops.MXFP4)
            got, got_sb = cache.load_mxfp4(pool, slots, 64, 128)
            want = packed if sgn > 0 else packed ^ np.uint8(0x88)
            if not np.array_equal(got, want):
                pytest.fail(f"bits {c0:#x}.. sign {sgn} (packed bytes, two inputs each): " + _first_diff(got, want))
            np.testing.assert_array_equal(got_sb, sb)


# ----------------------------------------------------------------------------------
# bf16 inputs: every pattern
# ----------------------------------------------------------------------------------
def _all_bf16() -> torch.Tensor:
    """Every non-NaN bf16 pattern, in pattern order."""
    b = np.arange(1 << 16, dtype=np.uint32)
    keep = ((b >> 7) & 0xFF) != 0xFF
    keep |= (b & 0x7F) == 0  # +-inf
    return torch.from_numpy((b[keep] << 16).view(np.float32)).to(torch.bfloat16)


def test_q_fp8_every_bf16_pattern():
    x = _all_bf16()
    rows = torch.cat([x, torch.zeros((-x.numel()) % 128, dtype=torch.bfloat16)]).view(-1, 128)
    got = ops.idx_q_quant(rows.view(-1, 1, 128).to(DEV), ops.FP8)[0].view(-1, 128).cpu().numpy()
    want = formats.quantize_fp8_noscale(rows.float().numpy())
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("anchor_bits", [0x40C0, 0x0140, 0x7F7F], ids=["e8m0_127", "e8m0_0", "e8m0_253"])
def test_q_mxfp4_every_bf16_pattern(anchor_bits):
    # every finite bf16 value at or below the anchor, in blocks the anchor scales
    x = _all_bf16().float().numpy()
    anchor = np.array([anchor_bits << 16], dtype=np.uint32).view(np.float32)[0]
    vals = x[np.isfinite(x) & (np.abs(x) <= anchor)]
    rows = _anchor_rows(anchor, vals, 32, 128)
    bf = torch.from_numpy(rows).to(torch.bfloat16)
    assert torch.equal(bf.float(), torch.from_numpy(rows))  # every value is a bf16 value
    out, sc = ops.idx_q_quant(bf.view(-1, 1, 128).to(DEV), ops.MXFP4)
    packed, sb = formats.quantize_mxfp4(rows)
    np.testing.assert_array_equal(out.view(-1, 64).cpu().numpy(), packed)
    np.testing.assert_array_equal(sc.view(-1).cpu().numpy(), formats.scales_to_int32(sb))
