"""Producers of the indexer's inputs: the query side (RoPE, quantisation, weight scale)
and the key side (RMSNorm, RoPE, quantisation into the cache).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Page ``vllm.models.deepseek_v41.amd.rocm``: ``rocm_mxfp4_indexer_q_quant`` hands the
queries, their positions, the rotary cos/sin table and the indexer weights to one fused
op, which returns the quantised queries (packed e2m1 with one int32 of e8m0 bytes per
head) and the weights multiplied by ``softmax_scale * n_head ** -0.5``;
``rocm_mxfp4_indexer_k_store`` hands the pre-norm keys, their positions, the cos/sin
table, the RMSNorm weight and epsilon and the slot mapping to one fused op that writes
the cache. The pages show these interfaces, not the bodies. Readings taken here:

* RoPE is the GPT-J rotation (pairs of adjacent channels) of the trailing ``rope_dim``
  channels of a 128-channel row; the leading ``D - rope_dim`` channels pass through.
  This is the convention of the inverse RoPE on page
  ``vllm.v1.attention.ops.rocm_aiter_mla_sparse`` (``_fused_inverse_rope_gptj`` and
  ``_inverse_rope_gptj_kernel``: non-rope channels first, pairs of adjacent lanes,
  a cos/sin table row of ``rope_dim`` values laid out as cos | sin). The forward
  rotation of a pair (a, b) is (a cos - b sin, b cos + a sin); the page's inverse maps
  it back with (a cos + b sin, b cos - a sin).
* RMSNorm is x / sqrt(mean(x ** 2) + eps) * weight over the 128 channels of a key,
  applied before RoPE.
* Every key row carries its own position (for a compressed cache the caller passes
  the position of the stored key); the normalised, rotated key is then quantised by
  the K-store rules of ``formats``, and the query by the query rules.

Everything is computed in float64; the GPU computes in float32, so quantised codes can
differ where a value lies within float32 rounding of a code boundary, and the tests
allow exactly that.
"""

from __future__ import annotations

import numpy as np


def rope_gptj(x, positions, cos_sin, rope_dim: int) -> np.ndarray:
    """GPT-J RoPE on the trailing rope_dim channels of x [..., D]; positions broadcast
    against x's leading dims (one per row); cos_sin [max_position, rope_dim] holds
    cos of the rope_dim // 2 pair angles, then their sin."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    if rope_dim % 2 or not 0 <= rope_dim <= D:
        raise ValueError("rope_dim must be even and at most D")
    half = rope_dim // 2
    cs = np.asarray(cos_sin, dtype=np.float64)[np.asarray(positions)]
    c, s = cs[..., :half], cs[..., half:rope_dim]
    y = x.copy()
    lo = D - rope_dim
    a, b = x[..., lo::2], x[..., lo + 1::2]
    y[..., lo::2] = a * c - b * s
    y[..., lo + 1::2] = b * c + a * s
    return y


def rms_norm(x, weight, eps: float) -> np.ndarray:
    """x / sqrt(mean(x ** 2) + eps) * weight over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + float(eps)) * np.asarray(weight, dtype=np.float64)


def k_norm_rope(k, positions, cos_sin, rope_dim: int, weight, eps: float) -> np.ndarray:
    """The key the store quantises: RMSNorm, then RoPE at the key's position."""
    return rope_gptj(rms_norm(k, weight, eps), np.asarray(positions), cos_sin, rope_dim)


def q_rope(q, positions, cos_sin, rope_dim: int) -> np.ndarray:
    """The query the quantiser sees: q [T, H, D] rotated at each token's position."""
    return rope_gptj(q, np.asarray(positions)[:, None], cos_sin, rope_dim)


def scale_weights(w, scale: float) -> np.ndarray:
    """The scored weights: w * scale, one float32 rounding of the exact product (the
    product of two float32 numbers is exact in float64)."""
    return (np.asarray(w, dtype=np.float32).astype(np.float64) * np.float64(np.float32(scale))).astype(np.float32)


def rope_table(max_position: int, rope_dim: int, base: float = 10000.0) -> np.ndarray:
    """A cos | sin table of the usual geometric frequencies, float64
    [max_position, rope_dim]: angle(p, i) = p * base ** (-2 i / rope_dim)."""
    half = rope_dim // 2
    inv = base ** (-np.arange(half, dtype=np.float64) * 2.0 / rope_dim)
    ang = np.arange(max_position, dtype=np.float64)[:, None] * inv[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1)
