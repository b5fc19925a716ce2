"""Pins for the oracle's vocabulary entropy and argmax (CPU).

Closed forms: a one-hot distribution has entropy 0, a uniform one ln V, and a
two-level distribution (k logits at a, V - k at b) has
H = -k p1 ln p1 - (V - k) p2 ln p2 with p1 = e^a / Z, p2 = e^b / Z. Sampled rows
agree with a 50-digit mpmath evaluation and with scipy.stats.entropy.
"""

import mpmath
import numpy as np
import pytest
import scipy.stats

from oracle import vocab_entropy_argmax


def test_one_hot_is_zero():
    z = np.full((3, 151936), -np.inf)
    z[0, 7] = 0.0
    z[1, 151935] = 5.0
    z[2, 0] = -3.0
    H, a = vocab_entropy_argmax(z)
    assert np.array_equal(H, np.zeros(3))
    assert a.tolist() == [7, 151935, 0]
    spike = np.zeros(1000)
    spike[3] = 1e4
    H, a = vocab_entropy_argmax(spike)
    assert H == 0.0 and a == 3


@pytest.mark.parametrize("V", [2, 512, 151936, 152064])
def test_uniform_is_log_v(V):
    H, a = vocab_entropy_argmax(np.full(V, 1.2345))
    assert abs(H - np.log(V)) <= 1e-12 * np.log(V)
    assert a == 0


@pytest.mark.parametrize("V,k,a,b", [(512, 1, 8.0, 0.0), (151936, 3, 10.0, -1.0),
                                     (1000, 500, 2.0, 1.0), (7, 6, -4.0, 3.0)])
def test_two_level_closed_form(V, k, a, b):
    z = np.full(V, b)
    z[:k] = a
    Z = k * np.exp(a) + (V - k) * np.exp(b)
    p1, p2 = np.exp(a) / Z, np.exp(b) / Z
    expect = -k * p1 * np.log(p1) - (V - k) * p2 * np.log(p2)
    H, arg = vocab_entropy_argmax(z)
    assert abs(H - expect) <= 1e-12 * max(1.0, expect)
    assert arg == (0 if a >= b else k)


def _mp_entropy(row):
    mpmath.mp.dps = 50
    zs = [mpmath.mpf(float(x)) for x in row]
    m = max(zs)
    es = [mpmath.e ** (x - m) for x in zs]
    s = mpmath.fsum(es)
    return float(-mpmath.fsum(e / s * mpmath.log(e / s) for e in es))


def test_matches_mpmath_and_scipy():
    rng = np.random.default_rng(0)
    rows = rng.normal(0, 2, size=(4, 2000))
    rows[1, 17] += 12.0
    rows[2, :] *= 10.0
    H, _ = vocab_entropy_argmax(rows)
    for i in range(rows.shape[0]):
        assert abs(H[i] - _mp_entropy(rows[i])) <= 1e-12 * max(1.0, H[i])
        p = np.exp(rows[i] - rows[i].max())
        assert abs(H[i] - scipy.stats.entropy(p)) <= 1e-11


def test_full_vocab_row_against_scipy():
    rng = np.random.default_rng(1)
    row = rng.normal(0, 2, size=151936).astype(np.float32).astype(np.float64)
    row[123] += 9.0
    H, a = vocab_entropy_argmax(row)
    p = np.exp(row - row.max())
    assert abs(H - scipy.stats.entropy(p)) <= 1e-10
    assert a == 123


def test_argmax_lowest_index_on_ties():
    z = np.array([[1.0, 3.0, 3.0, 2.0], [5.0, 5.0, 5.0, 5.0], [0.0, -1.0, 0.0, 0.0]])
    _, a = vocab_entropy_argmax(z)
    assert a.tolist() == [1, 0, 0]


def test_threaded_rows_are_bitwise_the_same():
    # rows are independent: dealing them to threads changes no bit
    z = np.random.default_rng(5).normal(0, 2, size=(7, 3, 4099))
    z[2, 1, 17] += 30.0
    H1, a1 = vocab_entropy_argmax(z)
    for workers in (2, 5, 64):
        H, a = vocab_entropy_argmax(z, workers=workers)
        assert np.array_equal(H, H1) and np.array_equal(a, a1)
