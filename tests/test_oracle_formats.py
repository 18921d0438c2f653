"""Pins of the oracle's number formats and quantisers against sources other than itself.

* e4m3 / e8m0 decoding: exhaustive against PyTorch's own float8 dtypes.
* e2m1 decoding: the 16-entry table typed in from the OCP Microscaling (MX) v1.0
  specification's FP4 (E2M1) element format.
* e4m3 rounding: PyTorch's float32 -> float8_e4m3fn cast (round to nearest even) and a
  brute-force nearest-value search.
* e2m1 rounding: hand-typed midpoint cases and a brute-force nearest-value search.
* e8m0 scale rule: a brute-force search for the smallest exponent that holds.
"""

import math

import numpy as np
import pytest
import torch

from oracle import formats

E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def test_e4m3_decode_exhaustive_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = formats.decode_e4m3(codes, allow_nan=True)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))
    assert np.isnan(ref).sum() == 2  # 0x7f and 0xff only
    with pytest.raises(ValueError):
        formats.decode_e4m3(np.array([0x7F], dtype=np.uint8))


def test_e8m0_decode_exhaustive_vs_torch():
    codes = np.arange(255, dtype=np.uint8)
    ours = formats.decode_e8m0(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)
    with pytest.raises(ValueError):
        formats.decode_e8m0(np.array([255], dtype=np.uint8))


def test_e2m1_decode_vs_spec_table():
    ours = formats.decode_e2m1(np.arange(16))
    assert np.array_equal(ours, np.array(E2M1_TABLE))
    assert np.array_equal(np.signbit(ours), np.signbit(np.array(E2M1_TABLE)))


def test_e2m1_pack_order():
    # element 2i in the low nibble of byte i
    nib = np.array([[1, 2, 3, 4]], dtype=np.uint8)
    assert formats.pack_e2m1(nib).tolist() == [[0x21, 0x43]]
    assert formats.unpack_e2m1(np.array([[0x21, 0x43]], dtype=np.uint8)).tolist() == [[1, 2, 3, 4]]


def test_scale_word_little_endian():
    b = np.array([[128, 127, 126, 1]], dtype=np.uint8)
    word = formats.scales_to_int32(b)
    assert int(word[0]) == 128 | (127 << 8) | (126 << 16) | (1 << 24)
    assert formats.scales_from_int32(word).tolist() == b.tolist()


def _all_e4m3_values():
    return [v for v in formats.decode_e4m3(np.arange(256, dtype=np.uint8), allow_nan=True)]


def test_e4m3_rounding_vs_torch_cast():
    rng = np.random.default_rng(7)
    # random magnitudes over the whole e4m3 range, plus every midpoint between
    # neighbouring codes and its float32 neighbours
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(50),
        np.ldexp(rng.random(50000), rng.integers(-14, 9, 50000)).astype(np.float32),
    ])
    mags = formats.decode_e4m3(np.arange(127, dtype=np.uint8))
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    mids = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1000))])
    x = np.concatenate([x, mids, -mids, np.float32([0.0, -0.0, 448.0, -448.0])])
    x = x[np.abs(x) <= 448]
    ours = formats.quant_e4m3(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_saturation():
    x = np.float32([448.0, 449.0, 464.0, 480.0, 1e30, -500.0, -1e38])
    assert formats.quant_e4m3(x).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


def test_e4m3_rounding_brute_force():
    rng = np.random.default_rng(8)
    x = np.ldexp(rng.random(3000) * 2 - 1, rng.integers(-12, 10, 3000)).astype(np.float32)
    table = _all_e4m3_values()
    ours = formats.quant_e4m3(x)
    for xi, c in zip(x.tolist(), ours.tolist()):
        best, bestd = None, None
        for code, v in enumerate(table):
            if math.isnan(v) or (code & 0x7F) == 0x7F:
                continue
            if (code >> 7) != (1 if math.copysign(1, xi) < 0 else 0):
                continue
            d = abs(abs(xi) - abs(v)) if abs(xi) <= 448 else abs(448 - abs(v))
            if bestd is None or d < bestd or (d == bestd and code % 2 == 0):
                best, bestd = code, d
        assert c == best, (xi, c, best)


def test_e2m1_rounding_midpoints():
    cases = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0,
             0.2: 0.0, 0.26: 0.5, 0.74: 0.5, 2.6: 3.0, 5.01: 6.0, 7.0: 6.0, 100.0: 6.0}
    for x, want in cases.items():
        for sgn in (1.0, -1.0):
            got = formats.decode_e2m1(formats.quant_e2m1(np.array([sgn * x])))[0]
            assert got == sgn * want, (sgn * x, got)


def test_e2m1_rounding_brute_force():
    rng = np.random.default_rng(9)
    x = rng.uniform(-7, 7, 5000)
    ours = formats.decode_e2m1(formats.quant_e2m1(x))
    for xi, got in zip(x.tolist(), ours.tolist()):
        cand = [v for v in E2M1_TABLE if (v < 0 or (v == 0 and math.copysign(1, v) < 0)) == (xi < 0)]
        dists = [abs(min(abs(xi), 6.0) - abs(v)) for v in cand]
        dmin = min(dists)
        near = [abs(v) for v, d in zip(cand, dists) if d == dmin]
        assert abs(got) in near
        if len(near) == 1:
            assert abs(got) == near[0]


def test_e8m0_rule_brute_force():
    rng = np.random.default_rng(10)
    amax = np.concatenate([
        np.ldexp(rng.random(2000) + 0.5, rng.integers(-140, 128, 2000)),
        np.ldexp(6.0, np.arange(-127, 128)),  # exact boundaries
        np.nextafter(np.ldexp(6.0, np.arange(-126, 127)), np.inf),
        np.nextafter(np.ldexp(6.0, np.arange(-126, 127)), 0),
        [0.0, 1e-45, float(np.finfo(np.float32).max)],
    ])
    amax = amax[amax <= float(np.finfo(np.float32).max)]
    got = formats.e8m0_block_bits(amax)
    for a, g in zip(amax.tolist(), got.tolist()):
        want = next(b for b in range(255) if a <= 6.0 * 2.0 ** (b - 127))
        assert g == want, (a, g, want)


def test_quantize_k_fp8_properties():
    rng = np.random.default_rng(11)
    k = rng.standard_normal((500, 128)).astype(np.float32)
    k[3] = 0.0
    codes, scale = formats.quantize_k_fp8(k)
    assert scale.dtype == np.float32
    assert scale[3] == 1.0 and not codes[3].any()
    amax = np.abs(k).max(axis=1)
    np.testing.assert_array_equal(scale[np.arange(500) != 3], (amax / np.float32(448))[np.arange(500) != 3])
    # the largest element of each row lands on +-448
    arg = np.abs(k).argmax(axis=1)
    top = codes[np.arange(500), arg]
    assert np.all((top[np.arange(500) != 3] & 0x7F) == 0x7E)
    # dequantised error within half an e4m3 spacing of the scaled value
    deq = formats.decode_e4m3(codes) * scale[:, None]
    rel = np.abs(deq - k) / np.maximum(np.abs(k), scale[:, None] * 2.0 ** -6)
    assert rel.max() <= 2.0 ** -4 + 1e-6


def test_quantize_mxfp4_properties():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((300, 128)).astype(np.float32) * np.float32(3.0)
    x[5, 32:64] = 0.0
    packed, bits = formats.quantize_mxfp4(x)
    assert packed.shape == (300, 64) and bits.shape == (300, 4)
    assert bits[5, 1] == 0
    deq = formats.decode_mxfp4(packed, bits)
    blocks = x.reshape(300, 4, 32).astype(np.float64)
    amax = np.abs(blocks).max(axis=2)
    scaled_amax = amax * np.ldexp(1.0, 127 - bits.astype(np.int64))
    nz = amax > 0
    assert np.all(scaled_amax[nz] <= 6.0) and np.all(scaled_amax[nz] > 3.0)
    # each element is within half a grid step (<= 1 at the top binade) of its scaled value
    err = np.abs(deq.reshape(300, 4, 32) - blocks) * np.ldexp(1.0, 127 - bits.astype(np.int64))[..., None]
    assert err.max() <= 1.0
