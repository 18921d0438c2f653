"""GPU parity of the quantisers: idx_q_quant and idx_k_store must match the oracle bit
for bit (byte work)."""

import numpy as np
import pytest
import torch

from oracle import cache, formats
from sparse_attention_indexer_mxfp4_amd import ops

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _special_values(rng, n):
    """Values that sit on rounding boundaries of e4m3 and e2m1, plus extremes."""
    mags = formats.decode_e4m3(np.arange(127, dtype=np.uint8))
    mids = (mags[:-1] + mags[1:]) / 2
    e2 = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0])
    base = np.concatenate([mags, mids, np.nextafter(mids.astype(np.float32), np.float32(1e9)), e2,
                           [0.0, 448.0, 449.0, 464.0, 1000.0, 1e30, 2.0 ** -10, 3 * 2.0 ** -10, 1e-40]])
    base = np.concatenate([base, -base]).astype(np.float32)
    return np.resize(rng.permutation(base), n).astype(np.float32)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_q_quant_fp8_bitexact(dtype):
    rng = np.random.default_rng(100)
    T, H = 37, 5
    q = rng.standard_normal((T, H, 128)).astype(np.float32) * np.float32(30)
    q[3] = _special_values(rng, H * 128).reshape(H, 128)
    qt = torch.from_numpy(q).to(dtype)
    q32 = qt.float().numpy()  # the exact values the kernel sees
    out, scale = ops.idx_q_quant(qt.to(DEV), ops.FP8)
    assert scale is None
    want = formats.quantize_fp8_noscale(q32)
    np.testing.assert_array_equal(out.cpu().numpy(), want)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_q_quant_mxfp4_bitexact(dtype):
    rng = np.random.default_rng(101)
    T, H = 29, 7
    q = rng.standard_normal((T, H, 128)).astype(np.float32)
    q *= np.ldexp(1.0, rng.integers(-20, 20, (T, H, 1))).astype(np.float32)
    q[2] = _special_values(rng, H * 128).reshape(H, 128) * np.float32(0.01)
    q[4, 1, 32:64] = 0.0
    q[5, 2] = 0.0
    qt = torch.from_numpy(q).to(dtype)
    q32 = qt.float().numpy()
    out, scale = ops.idx_q_quant(qt.to(DEV), ops.MXFP4)
    packed, bits = formats.quantize_mxfp4(q32)
    np.testing.assert_array_equal(out.cpu().numpy(), packed)
    np.testing.assert_array_equal(scale.cpu().numpy(), formats.scales_to_int32(bits))


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("page_size,stride_pad", [(64, 0), (16, 48), (128, 16)])
def test_k_store_bitexact(fmt, dtype, page_size, stride_pad):
    rng = np.random.default_rng(102)
    N, D = 300, 128
    num_pages = -(-N // page_size) + 2
    k = rng.standard_normal((N, D)).astype(np.float32)
    k *= np.ldexp(1.0, rng.integers(-8, 8, (N, 1))).astype(np.float32)
    k[7] = 0.0
    k[11] = _special_values(rng, D) * np.float32(0.5)
    kt = torch.from_numpy(k).to(dtype)
    k32 = kt.float().numpy()
    slots = rng.permutation(num_pages * page_size)[:N].astype(np.int64)
    slots[::17] = -1  # padding entries are skipped
    pb = (cache.fp8_page_bytes if fmt == "fp8" else cache.mxfp4_page_bytes)(page_size, D)
    pool0 = rng.integers(0, 256, (num_pages, pb + stride_pad)).astype(np.uint8)  # untouched bytes must survive
    want = pool0.copy()
    if fmt == "fp8":
        codes, sc = formats.quantize_k_fp8(k32)
        cache.store_fp8(want, slots, codes, sc, page_size)
    else:
        packed, sb = formats.quantize_mxfp4(k32)
        cache.store_mxfp4(want, slots, packed, sb, page_size)
    pool = torch.from_numpy(pool0).to(DEV)
    ops.idx_k_store(pool, ops.FP8 if fmt == "fp8" else ops.MXFP4, page_size, kt.to(DEV),
                    torch.from_numpy(slots).to(DEV))
    np.testing.assert_array_equal(pool.cpu().numpy(), want)


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("dtype,row_pad", [(torch.float32, 2), (torch.bfloat16, 3), (torch.float32, 4)])
def test_k_store_row_strides(fmt, dtype, row_pad):
    # key rows [N, 128] inside a wider buffer: padded rows, some not 16-byte aligned
    rng = np.random.default_rng(103)
    N, D, P = 77, 128, 16
    num_pages = -(-N // P) + 1
    big = rng.standard_normal((N, D + row_pad)).astype(np.float32)
    kt = torch.from_numpy(big).to(dtype).to(DEV)[:, 1:D + 1]  # offset by one element as well
    assert kt.stride(0) == D + row_pad
    k32 = kt.float().cpu().numpy()
    slots = rng.permutation(num_pages * P)[:N].astype(np.int64)
    pb = (cache.fp8_page_bytes if fmt == "fp8" else cache.mxfp4_page_bytes)(P, D)
    pool0 = np.zeros((num_pages, pb), dtype=np.uint8)
    want = pool0.copy()
    if fmt == "fp8":
        codes, sc = formats.quantize_k_fp8(k32)
        cache.store_fp8(want, slots, codes, sc, P)
    else:
        packed, sb = formats.quantize_mxfp4(k32)
        cache.store_mxfp4(want, slots, packed, sb, P)
    pool = torch.from_numpy(pool0).to(DEV)
    ops.idx_k_store(pool, ops.FP8 if fmt == "fp8" else ops.MXFP4, P, kt, torch.from_numpy(slots).to(DEV))
    np.testing.assert_array_equal(pool.cpu().numpy(), want)


def test_k_store_empty_is_noop():
    pool = torch.zeros((2, 8448), dtype=torch.uint8, device=DEV)
    ops.idx_k_store(pool, ops.FP8, 64, torch.zeros((0, 128), device=DEV), torch.zeros(0, dtype=torch.int64, device=DEV))
    assert int(pool.sum()) == 0
