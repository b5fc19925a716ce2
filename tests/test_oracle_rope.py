"""Pins for the oracle's RoPE at logical positions (CPU).

RoFormer's rotary embedding (mlsanity.com page on WeDLM, "Builds on") rotates
coordinate pairs by position-proportional angles, so a query-key dot product
depends only on the position difference; the WeDLM pages rely on this to keep
logical positions through the reordering (hyper.ai summary, "Method").
Pins: identity at t = 0, norm preservation, composition, the D = 2 complex
multiplication special case, closed-form angles for the rotate-half pairing,
and the relative-position (shift) invariance.
"""

import numpy as np

from oracle import rope_frequencies, rope_rotate


def test_frequencies_closed_form():
    w = rope_frequencies(4, 10000.0)
    assert np.allclose(w, [1.0, 0.01], rtol=0, atol=1e-15)
    w = rope_frequencies(128, 1e6)
    assert w[0] == 1.0
    assert abs(w[64 - 1] - 1e6 ** (-126 / 128)) < 1e-18


def test_identity_at_zero_and_norm():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 3, 128))
    assert np.array_equal(rope_rotate(x, np.zeros((5, 3)), 1e6), x)
    t = rng.integers(0, 40000, size=(5, 3))
    y = rope_rotate(x, t, 1e6)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)


def test_composition():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 64))
    a = rng.integers(0, 5000, size=7)
    b = rng.integers(0, 5000, size=7)
    lhs = rope_rotate(rope_rotate(x, a, 1e4), b, 1e4)
    rhs = rope_rotate(x, a + b, 1e4)
    assert np.allclose(lhs, rhs, atol=1e-10)


def test_d2_is_complex_multiplication():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((50, 2))
    t = rng.integers(0, 1000, size=50)
    z = (x[:, 0] + 1j * x[:, 1]) * np.exp(1j * t)   # omega_0 = theta^0 = 1
    y = rope_rotate(x, t, 1e4)
    assert np.allclose(y[:, 0], z.real, atol=1e-12)
    assert np.allclose(y[:, 1], z.imag, atol=1e-12)


def test_rotate_half_pairing_closed_form():
    # D = 4, theta = 1e4: dims (0, 2) rotate at omega 1, dims (1, 3) at 0.01.
    e1 = np.array([0.0, 1.0, 0.0, 0.0])
    y = rope_rotate(e1, 100, 1e4)        # angle 100 * 0.01 = 1 rad on pair (1, 3)
    assert np.allclose(y, [0.0, np.cos(1.0), 0.0, np.sin(1.0)], atol=1e-15)
    e0 = np.array([1.0, 0.0, 0.0, 0.0])
    y = rope_rotate(e0, 3, 1e4)          # angle 3 rad on pair (0, 2)
    assert np.allclose(y, [np.cos(3.0), 0.0, np.sin(3.0), 0.0], atol=1e-15)


def test_dot_product_depends_on_position_difference():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((20, 128))
    k = rng.standard_normal((20, 128))
    s = rng.integers(0, 40000, size=20)
    t = rng.integers(0, 40000, size=20)
    base = np.sum(rope_rotate(q, s, 1e6) * rope_rotate(k, t, 1e6), axis=-1)
    for c in (1, 17, 12345):
        shifted = np.sum(rope_rotate(q, s + c, 1e6) * rope_rotate(k, t + c, 1e6), axis=-1)
        assert np.allclose(shifted, base, rtol=1e-10, atol=1e-10)
