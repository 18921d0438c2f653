"""GPU parity of the fused producers: idx_k_norm_rope_store (RMSNorm + RoPE + K store)
and idx_q_rope_quant (RoPE + quantisation + weight scale) against the oracle.

The oracle computes the normalised, rotated values in float64; the GPU in float32.
A quantised code is accepted when it equals the oracle's rounding of the exact value
or lies as close to that value as the oracle's code does, give or take 1e-6 of the
row's largest magnitude (a near-tie that float32 rounding may resolve either way: a
rotated value can come from cancelling terms as large as the row's maximum, so its
float32 error is relative to that maximum, not to itself). That slack is far below
the spacing of any e4m3 or e2m1 code, so a wrong code still fails. A block or row
scale is accepted when it is the oracle's rule applied to the exact maximum give or
take float32 rounding. The scaled weights are one float32 multiply and must match
bit for bit."""

import numpy as np
import pytest
import torch

from oracle import cache, formats, producers
from sparse_attention_indexer_mxfp4_amd import ops

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
D = 128


def _slack(exact):
    """1e-6 of each row's largest magnitude, broadcast over the row."""
    return 1e-6 * np.broadcast_to(np.max(np.abs(exact), axis=-1, keepdims=True), exact.shape)


def _check_e4m3(codes, exact, what):
    """codes: GPU e4m3 bytes for the exact values `exact` (same shape, rows last)."""
    want = formats.quant_e4m3(exact)
    same = codes == want
    if not same.all():
        got_err = np.abs(formats.decode_e4m3(codes[~same]) - exact[~same])
        best_err = np.abs(formats.decode_e4m3(want[~same]) - exact[~same])
        assert np.all(got_err <= best_err + _slack(exact)[~same]), f"{what}: e4m3 code off"
    assert same.mean() > 0.999, f"{what}: too many near-ties ({(~same).sum()})"


def _check_e2m1(nibbles, exact, what):
    want = formats.quant_e2m1(exact)
    same = nibbles == want
    if not same.all():
        got_err = np.abs(formats.decode_e2m1(nibbles[~same]) - exact[~same])
        best_err = np.abs(formats.decode_e2m1(want[~same]) - exact[~same])
        assert np.all(got_err <= best_err + _slack(exact)[~same]), f"{what}: e2m1 code off"
    assert same.mean() > 0.999, f"{what}: too many near-ties ({(~same).sum()})"


def _check_mx(packed, bits, y, what):
    """packed [..., 64] e2m1 bytes and e8m0 bytes [..., 4] for exact rows y [..., 128]."""
    blocks = y.reshape(y.shape[:-1] + (4, 32))
    amax = np.max(np.abs(blocks), axis=-1)
    lo = formats.e8m0_block_bits(amax * (1 - 1e-6))
    hi = formats.e8m0_block_bits(amax * (1 + 1e-6))
    b = bits.astype(np.int64)
    assert np.all((b >= lo) & (b <= hi)), f"{what}: block scale off"
    scaled = blocks * np.ldexp(1.0, 127 - b)[..., None]
    _check_e2m1(formats.unpack_e2m1(packed), scaled.reshape(y.shape), what)


def _table(max_pos, rope_dim):
    return producers.rope_table(max_pos, rope_dim).astype(np.float32)


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("rope_dim", [64, 0, 128])
def test_k_norm_rope_store(fmt, dtype, rope_dim):
    rng = np.random.default_rng(201 + rope_dim)
    N, P, maxp = 300, 64, 4096
    num_pages = -(-N // P) + 2
    k = (rng.standard_normal((N, D)) * rng.uniform(0.1, 30.0, (N, 1))).astype(np.float32)
    kt = torch.from_numpy(k).to(dtype)
    k64 = kt.float().numpy().astype(np.float64)
    pos = rng.integers(0, maxp, N).astype(np.int64)
    pos[:3] = [0, maxp - 1, maxp + 50]  # the last one is clamped to maxp - 1
    table = _table(maxp, rope_dim) if rope_dim else np.zeros((1, 0), np.float32)
    wgt = rng.uniform(0.5, 1.5, D).astype(np.float32)
    eps = 1e-6
    slots = rng.permutation(num_pages * P)[:N].astype(np.int64)
    slots[::23] = -1
    pb = (cache.fp8_page_bytes if fmt == "fp8" else cache.mxfp4_page_bytes)(P, D)
    pool = torch.zeros((num_pages, pb), dtype=torch.uint8, device=DEV)
    ops.idx_k_norm_rope_store(pool, ops.FP8 if fmt == "fp8" else ops.MXFP4, P, kt.to(DEV),
                              torch.from_numpy(slots).to(DEV),
                              torch.from_numpy(pos).to(DEV) if rope_dim else None,
                              torch.from_numpy(table).to(DEV) if rope_dim else None, rope_dim,
                              torch.from_numpy(wgt).to(DEV), eps)
    got = pool.cpu().numpy()
    live = slots >= 0
    posc = np.minimum(pos, maxp - 1)
    if rope_dim:
        y = producers.k_norm_rope(k64, posc, table.astype(np.float64), rope_dim, wgt.astype(np.float64), eps)
    else:
        y = producers.rms_norm(k64, wgt.astype(np.float64), eps)
    y = y[live]
    if fmt == "fp8":
        codes, scales = cache.load_fp8(got, slots[live], P, D)
        amax = np.max(np.abs(y), axis=1)
        np.testing.assert_allclose(scales, amax / 448.0, rtol=2e-6)
        _check_e4m3(codes, y / scales.astype(np.float64)[:, None], "k fp8")
    else:
        packed, bits = cache.load_mxfp4(got, slots[live], P, D)
        _check_mx(packed, bits, y, "k mxfp4")
    # padding slots left the pool untouched elsewhere: every byte not owned by a live
    # key is still zero
    owned = np.zeros_like(got, dtype=bool)
    page, entry = slots[live] // P, slots[live] % P
    if fmt == "fp8":
        vo, so = cache._fp8_offsets(P, D, entry)
    else:
        vo, so = cache._mxfp4_offsets(P, D, entry)
    owned[page[:, None], vo] = True
    owned[page[:, None], so] = True
    assert not got[~owned].any()


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_q_rope_quant(fmt, dtype):
    rng = np.random.default_rng(301)
    T, H, rope_dim, maxp = 37, 64, 64, 2048
    q = (rng.standard_normal((T, H, D)) * 2.0).astype(np.float32)
    qt = torch.from_numpy(q).to(dtype)
    q64 = qt.float().numpy().astype(np.float64)
    pos = rng.integers(0, maxp, T).astype(np.int64)
    table = _table(maxp, rope_dim)
    w = rng.standard_normal((T, H)).astype(np.float32)
    scale = np.float32(0.125 * H ** -0.5)
    out, qs, w_out = ops.idx_q_rope_quant(qt.to(DEV), ops.FP8 if fmt == "fp8" else ops.MXFP4,
                                          torch.from_numpy(pos).to(DEV), torch.from_numpy(table).to(DEV), rope_dim,
                                          torch.from_numpy(w).to(DEV), float(scale))
    y = producers.q_rope(q64, pos, table.astype(np.float64), rope_dim)
    np.testing.assert_array_equal(w_out.cpu().numpy(), producers.scale_weights(w, scale))
    if fmt == "fp8":
        _check_e4m3(out.cpu().numpy(), y, "q fp8")
    else:
        bits = formats.scales_from_int32(qs.cpu().numpy())
        _check_mx(out.cpu().numpy(), bits, y, "q mxfp4")


def test_q_rope_without_rope_matches_plain_quantiser():
    # rope_dim 0 leaves the query as it is: the fused op must reproduce idx_q_quant
    rng = np.random.default_rng(302)
    q = torch.from_numpy(rng.standard_normal((9, 16, D)).astype(np.float32)).to(DEV)
    w = torch.ones((9, 16), dtype=torch.float32, device=DEV)
    for fmt in (ops.FP8, ops.MXFP4):
        a, sa = ops.idx_q_quant(q, fmt)
        b, sb, _ = ops.idx_q_rope_quant(q, fmt, None, None, 0, w, 1.0)
        assert torch.equal(a, b)
        if sa is not None:
            assert torch.equal(sa, sb)
