"""Number formats of the indexer, decoded and encoded by their bit-field definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* e4m3 is the OCP ``float8_e4m3fn`` format (gfx950 uses OCP fp8, not the FNUZ variant
  of gfx942: page ``vllm.v1.attention.ops.rocm_aiter_mla_sparse``, the comment in
  ``_rocm_sparse_attn_decode_ragged_triton`` on the ~1.87x FNUZ/OCP scale ratio). It is
  the dtype of q and k in ``fp8_mqa_logits_torch`` and of the paged fp8 cache in
  ``rocm_fp8_paged_mqa_logits`` (same page).
* e2m1 (fp4) packed two per byte and e8m0 (unsigned power-of-two exponent, bias 127)
  per 32 values are the MXFP4 formats of the query and the key cache (page
  ``vllm.v1.attention.ops.rocm_paged_mxfp4_indexer``, ``rocm_mxfp4_sparse_attn_indexer``:
  "packed e2m1", "ue8m0 bytes ... one int32 per head at D = 128"). The bias 127 is the
  one the e8m0 rule ``_mxfp8_scale_bits`` uses (page
  ``vllm.v1.attention.ops.rocm_aiter_mla_sparse``).

Decoders return float64; every value of these formats is exact in float64.

Quantisers (the K store and the input preparation):

* ``quant_e4m3`` rounds to the nearest finite e4m3 value, ties to the even code, and
  saturates at +-448.
* ``quant_e2m1`` rounds to the nearest e2m1 value, ties to the even code, saturating
  at +-6.
* ``e8m0_block_bits`` is the smallest exponent byte b in [0, 254] with
  amax <= 6 * 2**(b - 127): the exact form of the ceil(log2(amax / max_code)) + 127
  rule of ``_mxfp8_scale_bits`` with the e2m1 maximum 6 in place of 448.
* ``quantize_k_fp8`` is the per-token fp32 absmax scale (amax / 448, 1.0 for an
  all-zero row), then e4m3 of the fp32 quotient k / scale.
* ``quantize_mxfp4`` scales each 32-value block by 2**(127 - b) (a multiply by the
  reciprocal, as ``_mxfp8_quantize_rows`` does) and rounds to e2m1; element 2i goes
  to the low nibble of byte i.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E2M1_MAX = 6.0
MX_BLOCK = 32


# ----------------------------------------------------------------------------------
# decoders
# ----------------------------------------------------------------------------------
def decode_e4m3(codes, allow_nan: bool = False) -> np.ndarray:
    """e4m3fn byte -> float64. s = b>>7, e = (b>>3)&15, m = b&7.

    e = 0 is subnormal, (m/8) * 2**-6; e = 15, m = 7 is NaN (rejected unless
    ``allow_nan``); otherwise (1 + m/8) * 2**(e - 7).
    """
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = b >> 7
    e = (b >> 3) & 15
    m = b & 7
    nan = (e == 15) & (m == 7)
    if nan.any() and not allow_nan:
        raise ValueError("e4m3 NaN code in input")
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64)))
    v = np.where(s == 1, -mag, mag)
    return np.where(nan, np.nan, v)


def decode_e2m1(nibbles) -> np.ndarray:
    """e2m1 nibble -> float64. s = n>>3, e = (n>>1)&3, m = n&1.

    e = 0 is subnormal, m * 0.5; otherwise (1 + m/2) * 2**(e - 1).
    """
    n = np.asarray(nibbles, dtype=np.int64) & 15
    s = n >> 3
    e = (n >> 1) & 3
    m = n & 1
    mag = np.where(e == 0, m * 0.5, np.ldexp(1.0 + m / 2.0, (e - 1)))
    return np.where(s == 1, -mag, mag)


def decode_e8m0(codes) -> np.ndarray:
    """e8m0 byte -> 2**(b - 127) as float64; 255 is NaN and rejected."""
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    if (b == 255).any():
        raise ValueError("e8m0 NaN code in input")
    return np.ldexp(1.0, b - 127)


def unpack_e2m1(packed) -> np.ndarray:
    """[..., n] bytes -> [..., 2n] nibbles; element 2i is the low nibble of byte i."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


def pack_e2m1(nibbles) -> np.ndarray:
    """[..., 2n] nibbles -> [..., n] bytes; element 2i goes to the low nibble."""
    n = np.asarray(nibbles, dtype=np.uint8)
    return (n[..., 0::2] & 15) | ((n[..., 1::2] & 15) << 4)


def decode_mxfp4(packed, scale_bytes) -> np.ndarray:
    """MXFP4 row(s) -> float64 values: e2m1 value times 2**(e - 127) of its 32-block.

    ``packed`` is [..., D/2], ``scale_bytes`` is [..., D/32].
    """
    vals = decode_e2m1(unpack_e2m1(packed))
    sc = decode_e8m0(scale_bytes)
    D = vals.shape[-1]
    return (vals.reshape(vals.shape[:-1] + (D // MX_BLOCK, MX_BLOCK)) * sc[..., None]).reshape(vals.shape)


def scales_from_int32(words) -> np.ndarray:
    """One int32 per head -> its 4 e8m0 bytes; byte j (little-endian) is block j's."""
    w = np.asarray(words, dtype=np.int64) & 0xFFFFFFFF
    return np.stack([(w >> (8 * j)) & 0xFF for j in range(4)], axis=-1).astype(np.uint8)


def scales_to_int32(scale_bytes) -> np.ndarray:
    """[..., 4] e8m0 bytes -> one int32 per head, byte j in bits 8j..8j+7."""
    b = np.asarray(scale_bytes, dtype=np.uint8).astype(np.uint32)
    word = b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16) | (b[..., 3] << 24)
    return word.astype(np.uint32).view(np.int32)


# ----------------------------------------------------------------------------------
# round-to-nearest-even onto a small grid
# ----------------------------------------------------------------------------------
def _round_to_grid(x, mags: np.ndarray, max_code: int) -> np.ndarray:
    """Sign-magnitude code of the grid value nearest |x|, ties to the even code.

    ``mags`` are the non-negative magnitudes of codes 0..max_code, increasing. The
    midpoint test compares 2|x| with mags[lo] + mags[hi], both exact in float64 for
    these grids, so ties are found exactly. Magnitudes past the last grid value
    saturate to it.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("NaN cannot be quantised")
    a = np.abs(x)
    hi = np.searchsorted(mags, a, side="left")  # mags[hi-1] < a <= mags[hi]
    hi = np.minimum(hi, max_code)
    lo = np.maximum(hi - 1, 0)
    twice = 2.0 * a
    mid = mags[lo] + mags[hi]
    pick_hi = (twice > mid) | ((twice == mid) & (hi % 2 == 0))
    code = np.where(a >= mags[max_code], max_code, np.where(pick_hi, hi, lo))
    code = np.where(a == 0.0, 0, code)
    sign = np.signbit(x)
    return code.astype(np.int64), sign


_E4M3_MAGS = decode_e4m3(np.arange(127, dtype=np.uint8))  # codes 0x00..0x7e, increasing
_E2M1_MAGS = decode_e2m1(np.arange(8))  # 0, .5, 1, 1.5, 2, 3, 4, 6


def quant_e4m3(x) -> np.ndarray:
    """float -> e4m3fn byte: nearest finite value, ties to even, saturating at +-448."""
    code, sign = _round_to_grid(x, _E4M3_MAGS, 126)
    return (code | (sign.astype(np.int64) << 7)).astype(np.uint8)


def quant_e2m1(x) -> np.ndarray:
    """float -> e2m1 nibble: nearest value, ties to even, saturating at +-6."""
    code, sign = _round_to_grid(x, _E2M1_MAGS, 7)
    return (code | (sign.astype(np.int64) << 3)).astype(np.uint8)


# ----------------------------------------------------------------------------------
# scale rules and row quantisers
# ----------------------------------------------------------------------------------
def e8m0_block_bits(amax) -> np.ndarray:
    """Smallest b in [0, 254] with amax <= 6 * 2**(b - 127); 0 for amax = 0.

    A float log2 gives the estimate; exact comparisons against 6 * 2**(b - 127)
    (exact in float64) then move it to the smallest b that holds.
    """
    a = np.asarray(amax, dtype=np.float64)
    with np.errstate(divide="ignore"):
        est = np.where(a > 0, np.ceil(np.log2(np.where(a > 0, a, 1.0) / E2M1_MAX)) + 127, 0)
    b = np.clip(est, 0, 254).astype(np.int64)
    for _ in range(2):
        b = np.where((a > np.ldexp(E2M1_MAX, b - 127)) & (b < 254), b + 1, b)
    for _ in range(2):
        b = np.where((b > 0) & (a <= np.ldexp(E2M1_MAX, b - 1 - 127)), b - 1, b)
    return b.astype(np.uint8)


def quantize_k_fp8(k) -> tuple[np.ndarray, np.ndarray]:
    """Per-token fp8 K: scale = amax / 448 in fp32 (1.0 if amax = 0),
    code = e4m3(fp32(k / scale)) with IEEE fp32 division. k is [N, D] (fp32 or bf16
    values, held exactly in fp32)."""
    k32 = np.asarray(k, dtype=np.float32)
    amax = np.max(np.abs(k32), axis=-1)
    scale = np.where(amax == 0, np.float32(1.0), amax / np.float32(E4M3_MAX)).astype(np.float32)
    quot = (k32 / scale[..., None]).astype(np.float32)
    return quant_e4m3(quot), scale


def quantize_fp8_noscale(x) -> np.ndarray:
    """q for the fp8 paths: e4m3 of the value itself (the fp8 API carries no q scale)."""
    return quant_e4m3(np.asarray(x, dtype=np.float32))


def quantize_mxfp4(x) -> tuple[np.ndarray, np.ndarray]:
    """[..., D] -> (packed e2m1 [..., D/2] uint8, e8m0 bytes [..., D/32] uint8)."""
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    D = x64.shape[-1]
    blocks = x64.reshape(x64.shape[:-1] + (D // MX_BLOCK, MX_BLOCK))
    bits = e8m0_block_bits(np.max(np.abs(blocks), axis=-1))
    scaled = blocks * np.ldexp(1.0, 127 - bits.astype(np.int64))[..., None]
    nib = quant_e2m1(scaled).reshape(x64.shape)
    return pack_e2m1(nib), bits
