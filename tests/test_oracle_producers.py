"""Pins of the oracle's producers (RoPE, RMSNorm, weight scaling): hand-worked values,
closed forms and invariants that a wrong sign, index or order would break."""

import json
import os

import numpy as np
import pytest

from oracle import producers

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "handworked_rope_norm.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_rope_handworked():
    g = _golden()["rope"]
    y = producers.rope_gptj(np.array(g["x"], float), g["position"], np.array(g["table"], float), g["rope_dim"])
    np.testing.assert_array_equal(y, np.array(g["want"], float))


def test_rms_norm_handworked():
    g = _golden()["rms_norm"]
    y = producers.rms_norm(np.array(g["x"], float), np.array(g["weight"], float), g["eps"])
    np.testing.assert_allclose(y, np.array(g["want"], float), rtol=0, atol=1e-15)


def test_weight_scale_handworked():
    g = _golden()["weights"]
    s = g["softmax_scale"] * g["n_head"] ** -0.5
    assert float(producers.scale_weights(np.float32(g["w"]), s)) == g["want"]


def test_weight_scale_is_one_float32_multiply():
    rng = np.random.default_rng(0)
    w = rng.standard_normal(1000).astype(np.float32)
    s = np.float32(0.088388347648318)
    np.testing.assert_array_equal(producers.scale_weights(w, s), w * s)


@pytest.mark.parametrize("rope_dim", [2, 64, 128])
def test_rope_keeps_pair_norms_and_passes_nope(rope_dim):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((50, 128))
    pos = rng.integers(0, 4096, 50)
    t = producers.rope_table(4096, rope_dim)
    y = producers.rope_gptj(x, pos, t, rope_dim)
    lo = 128 - rope_dim
    np.testing.assert_array_equal(y[:, :lo], x[:, :lo])
    nx = x[:, lo::2] ** 2 + x[:, lo + 1::2] ** 2
    ny = y[:, lo::2] ** 2 + y[:, lo + 1::2] ** 2
    np.testing.assert_allclose(ny, nx, rtol=1e-12)


def test_rope_position_zero_and_empty_rope_are_identity():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 128))
    t = producers.rope_table(16, 64)
    np.testing.assert_allclose(producers.rope_gptj(x, np.zeros(4, int), t, 64), x, rtol=0, atol=0)
    np.testing.assert_array_equal(producers.rope_gptj(x, np.ones(4, int), np.zeros((2, 0)), 0), x)


def test_rope_angle_addition():
    # rotating by position p1 then p2 equals rotating by p1 + p2 (angles add)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((20, 128))
    t = producers.rope_table(8192, 64)
    p1 = rng.integers(0, 4000, 20)
    p2 = rng.integers(0, 4000, 20)
    y = producers.rope_gptj(producers.rope_gptj(x, p1, t, 64), p2, t, 64)
    np.testing.assert_allclose(y, producers.rope_gptj(x, p1 + p2, t, 64), rtol=0, atol=1e-9)


def test_rope_inverted_by_the_pages_inverse():
    # the page's inverse: (a cos + b sin, b cos - a sin) restores the input
    rng = np.random.default_rng(4)
    x = rng.standard_normal((10, 128))
    t = producers.rope_table(512, 64)
    pos = rng.integers(0, 512, 10)
    y = producers.rope_gptj(x, pos, t, 64)
    c, s = t[pos, :32], t[pos, 32:]
    a, b = y[:, 64::2], y[:, 65::2]
    back = y.copy()
    back[:, 64::2] = a * c + b * s
    back[:, 65::2] = b * c - a * s
    np.testing.assert_allclose(back, x, rtol=0, atol=1e-12)


def test_rope_table_matches_angles():
    t = producers.rope_table(3, 4, base=100.0)
    # pair i frequency 100^(-2i/4): 1 and 1/10
    ang = np.array([[0, 0], [1, 0.1], [2, 0.2]])
    np.testing.assert_allclose(t, np.concatenate([np.cos(ang), np.sin(ang)], axis=1), rtol=0, atol=1e-15)


def test_rms_norm_invariants():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((30, 128)) * rng.uniform(0.01, 100, (30, 1))
    eps = 1e-6
    y = producers.rms_norm(x, np.ones(128), eps)
    ms = np.mean(x * x, axis=1)
    np.testing.assert_allclose(np.mean(y * y, axis=1), ms / (ms + eps), rtol=1e-12)
    # with eps = 0 the norm is homogeneous of degree 0 (sign kept)
    np.testing.assert_allclose(producers.rms_norm(-3.5 * x, np.ones(128), 0.0), -producers.rms_norm(x, np.ones(128), 0.0),
                               rtol=1e-13)
    wgt = rng.standard_normal(128)
    np.testing.assert_allclose(producers.rms_norm(x, wgt, eps), y * wgt, rtol=1e-13)


def test_norm_then_rope_order():
    # RMSNorm comes first: rotating first would change nothing only if the weight were
    # uniform; a non-uniform weight tells the two orders apart
    rng = np.random.default_rng(6)
    x = rng.standard_normal((5, 128))
    wgt = np.linspace(0.5, 2.0, 128)
    t = producers.rope_table(64, 64)
    pos = rng.integers(1, 64, 5)
    got = producers.k_norm_rope(x, pos, t, 64, wgt, 1e-6)
    want = producers.rope_gptj(producers.rms_norm(x, wgt, 1e-6), pos, t, 64)
    np.testing.assert_array_equal(got, want)
    other = producers.rms_norm(producers.rope_gptj(x, pos, t, 64), wgt, 1e-6)
    assert not np.allclose(got, other)


def test_q_rope_uses_each_tokens_position_for_all_heads():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((3, 4, 128))
    t = producers.rope_table(32, 64)
    pos = np.array([5, 0, 31])
    y = producers.q_rope(q, pos, t, 64)
    for i in range(3):
        for h in range(4):
            np.testing.assert_array_equal(y[i, h], producers.rope_gptj(q[i, h], pos[i], t, 64))
