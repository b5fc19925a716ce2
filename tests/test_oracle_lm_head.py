"""Pins for the oracle's vocabulary projection and its entropy selection (CPU).

The projection is pinned without re-calling its matrix product: a one-hot
hidden state must pick out one column of the projection (so rows and columns
cannot be swapped), a pure-Python triple loop with exact summation must agree
on a small random case, projections built along one direction give logits with
a closed-form two-level entropy, and a zero hidden state gives the uniform
distribution (entropy ln V, argmax 0).
"""

import math

import numpy as np

from oracle import lm_head_select, vocab_projection


def test_one_hot_hidden_selects_a_column():
    rng = np.random.default_rng(1)
    V, Hd = 7, 5
    w = rng.standard_normal((V, Hd))
    for k in range(Hd):
        h = np.zeros(Hd)
        h[k] = 1.0
        z = vocab_projection(h, w)
        assert z.shape == (V,)
        assert np.array_equal(z, w[:, k])
    # a non-square projection cannot be applied the other way round
    h = np.zeros((2, 3, Hd))
    h[1, 2, 4] = 2.0
    z = vocab_projection(h, w)
    assert z.shape == (2, 3, V)
    assert np.array_equal(z[1, 2], 2.0 * w[:, 4]) and not z[0].any()


def test_brute_force_small():
    rng = np.random.default_rng(2)
    B, W, Hd, V = 2, 3, 4, 6
    h = rng.standard_normal((B, W, Hd))
    w = rng.standard_normal((V, Hd))
    z = vocab_projection(h, w)
    for b in range(B):
        for i in range(W):
            for v in range(V):
                exact = math.fsum(float(h[b, i, k]) * float(w[v, k]) for k in range(Hd))
                assert abs(z[b, i, v] - exact) <= 1e-14 * max(1.0, abs(exact))


def test_two_level_projection_closed_form():
    # rows of the projection along one unit direction u: k rows give logit a,
    # the others b, for a hidden state h = u
    rng = np.random.default_rng(3)
    V, Hd, k, a, b = 1000, 64, 3, 9.0, 1.5
    u = rng.standard_normal(Hd)
    u /= np.linalg.norm(u)
    w = np.outer(np.where(np.arange(V) < k, a, b), u)
    out = lm_head_select(u[None, None, :], w, np.zeros((1, 1), bool), 0.1, 1.0)
    Z = k * math.exp(a) + (V - k) * math.exp(b)
    p1, p2 = math.exp(a) / Z, math.exp(b) / Z
    expect = -k * p1 * math.log(p1) - (V - k) * p2 * math.log(p2)
    assert abs(out["entropy"][0, 0] - expect) <= 1e-12 * expect
    assert out["argmax"][0, 0] == 0


def test_zero_hidden_is_uniform():
    V, Hd, W = 5000, 128, 4
    w = np.random.default_rng(4).standard_normal((V, Hd))
    filled = np.array([[True, False, False, True]])
    out = lm_head_select(np.zeros((1, W, Hd)), w, filled, 0.1, 100.0)
    assert np.allclose(out["entropy"], math.log(V), rtol=0, atol=1e-12)
    assert (out["argmax"] == 0).all()
    # every mask slot clears a threshold above ln V + lambda * (W - 1)
    assert out["select"][0]["selected"].tolist() == [False, True, True, False]
