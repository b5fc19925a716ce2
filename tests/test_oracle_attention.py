"""Pins for the oracle's window attention (CPU).

What the pages fix (hyper.ai summary of WeDLM, "Method"; sai.science review,
"Summary" and "Strengths"):
  (1) reorder-then-causal attention equals attention under the explicit
      visibility rule (each mask slot sees every observed token, observed
      tokens see earlier observed tokens) - Form R against Form M over every
      filled pattern of a W = 8 window;
  (2) the committed prefix's attention is a plain causal computation over
      [prefix ; committed tokens], and its cache rows are a plain append;
  (3) shifting every logical position by a constant leaves the result
      unchanged (RoPE depends on position differences only).
Special cases that reduce to library routines: an all-filled window is
ordinary causal attention with a KV cache (torch's scaled_dot_product_attention
in float64 on the CPU, with GQA), L = 0 and W = 1 returns v, q = 0 averages
the visible values.
"""

import itertools

import numpy as np
import pytest
import torch

from oracle import (rope_rotate, topological_reorder, window_attention_masked,
                    window_attention_reordered)


def _inputs(rng, L, W, Hq, Hkv, D):
    return (rng.standard_normal((W, Hq, D)), rng.standard_normal((W, Hkv, D)),
            rng.standard_normal((W, Hkv, D)), rng.standard_normal((L, Hkv, D)),
            rng.standard_normal((L, Hkv, D)))


def _form_r_in_slot_order(filled, q, k, v, kc, vc, L, theta):
    r = topological_reorder(filled, L)
    perm, pos = r["perm"], r["pos"]
    qp = rope_rotate(q[perm], pos[:, None], theta)
    kp = rope_rotate(k[perm], pos[:, None], theta)
    out_phys = window_attention_reordered(qp, kp, v[perm], kc, vc)
    return out_phys[r["inv"]]


def _form_m(filled, q, k, v, kc, vc, L, theta):
    W = len(filled)
    slot_pos = L + np.arange(W)
    return window_attention_masked(rope_rotate(q, slot_pos[:, None], theta),
                                   rope_rotate(k, slot_pos[:, None], theta), v, filled, kc, vc)


def test_form_r_equals_form_m_every_pattern_tiny_shape():
    # one sequence, 2 query heads on 1 kv head, D = 64, theta 1e4, L = 40, W = 8
    rng = np.random.default_rng(0)
    L, W, Hq, Hkv, D, theta = 40, 8, 2, 1, 64, 1e4
    q, k, v, kc, vc = _inputs(rng, L, W, Hq, Hkv, D)
    worst = 0.0
    for bits in itertools.product([False, True], repeat=W):
        a = _form_r_in_slot_order(bits, q, k, v, kc, vc, L, theta)
        b = _form_m(bits, q, k, v, kc, vc, L, theta)
        worst = max(worst, float(np.max(np.abs(a - b))))
    assert worst <= 1e-12


def test_form_r_equals_form_m_gqa_random_patterns():
    rng = np.random.default_rng(1)
    for _ in range(20):
        W = int(rng.integers(1, 33))
        L = int(rng.integers(0, 70))
        Hkv = int(rng.integers(1, 4))
        g = int(rng.integers(1, 8))
        q, k, v, kc, vc = _inputs(rng, L, W, Hkv * g, Hkv, 16)
        filled = rng.random(W) < rng.random()
        if L == 0 and not filled.any() and W == 0:
            continue
        a = _form_r_in_slot_order(filled, q, k, v, kc, vc, L, 1e6)
        b = _form_m(filled, q, k, v, kc, vc, L, 1e6)
        assert np.max(np.abs(a - b)) <= 1e-12


def _sdpa_causal_with_prefix(qr, kr, v, kc, vc, g):
    """torch SDPA in float64: W queries after an L-token prefix, plain causal."""
    W, Hq, D = qr.shape
    L = kc.shape[0]
    keys = np.concatenate([kc, kr], axis=0)        # [L+W, Hkv, D]
    vals = np.concatenate([vc, v], axis=0)
    Q = torch.from_numpy(np.ascontiguousarray(qr.transpose(1, 0, 2)))[None]
    K = torch.from_numpy(np.ascontiguousarray(keys.transpose(1, 0, 2)))[None]
    V = torch.from_numpy(np.ascontiguousarray(vals.transpose(1, 0, 2)))[None]
    mask = torch.ones(W, L + W, dtype=torch.bool)
    mask[:, L:] = torch.tril(torch.ones(W, W, dtype=torch.bool))
    out = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask,
                                                           enable_gqa=(g > 1))
    return out[0].numpy().transpose(1, 0, 2)


@pytest.mark.parametrize("Hq,Hkv", [(2, 1), (8, 8), (28, 4), (32, 8)])
def test_all_filled_window_is_ordinary_causal_attention(Hq, Hkv):
    rng = np.random.default_rng(2)
    L, W, D, theta = 37, 16, 32, 1e6
    q, k, v, kc, vc = _inputs(rng, L, W, Hq, Hkv, D)
    filled = np.ones(W, bool)
    ours = _form_r_in_slot_order(filled, q, k, v, kc, vc, L, theta)
    pos = L + np.arange(W)
    ref = _sdpa_causal_with_prefix(rope_rotate(q, pos[:, None], theta),
                                   rope_rotate(k, pos[:, None], theta), v, kc, vc, Hq // Hkv)
    assert np.max(np.abs(ours - ref)) <= 1e-12


def test_single_token_no_prefix_returns_v():
    rng = np.random.default_rng(3)
    q, k, v, kc, vc = _inputs(rng, 0, 1, 6, 2, 8)
    out = window_attention_reordered(q, k, v, kc, vc)
    assert np.array_equal(out[0, :3], np.repeat(v[0, :1], 3, axis=0))
    assert np.array_equal(out[0, 3:], np.repeat(v[0, 1:], 3, axis=0))


def test_zero_query_averages_visible_values():
    rng = np.random.default_rng(4)
    L, W, D = 11, 6, 8
    _, k, v, kc, vc = _inputs(rng, L, W, 1, 1, D)
    q = np.zeros((W, 1, D))
    out = window_attention_reordered(q, k, v, kc, vc)
    for p in range(W):
        ref = np.concatenate([vc[:, 0], v[: p + 1, 0]]).mean(axis=0)
        assert np.allclose(out[p, 0], ref, atol=1e-14)


def test_committed_prefix_is_plain_causal_recompute():
    """Invariant (2): rows of the leading filled run equal a plain causal run."""
    rng = np.random.default_rng(5)
    L, W, Hq, Hkv, D, theta = 25, 12, 4, 2, 16, 1e4
    q, k, v, kc, vc = _inputs(rng, L, W, Hq, Hkv, D)
    for trial in range(20):
        filled = rng.random(W) < 0.6
        c = int(rng.integers(1, W + 1))
        filled[:c] = True
        if c < W:
            filled[c] = False
        r = topological_reorder(filled, L)
        assert r["run"] == c
        out_slot = _form_r_in_slot_order(filled, q, k, v, kc, vc, L, theta)
        pos = L + np.arange(c)
        qr = rope_rotate(q[:c], pos[:, None], theta)
        kr = rope_rotate(k[:c], pos[:, None], theta)
        plain = _sdpa_causal_with_prefix(qr, kr, v[:c], kc, vc, Hq // Hkv)
        assert np.max(np.abs(out_slot[:c] - plain)) <= 1e-12
        # the cache rows a commit appends are the plainly rotated keys of the run
        kp = rope_rotate(k[r["perm"]], r["pos"][:, None], theta)
        assert np.array_equal(kp[:c], kr)


def test_shift_of_all_positions_leaves_attention_unchanged():
    """Invariant (3): raw prefix keys rotated at 0..L-1, window at L..L+W-1, all + c."""
    rng = np.random.default_rng(6)
    L, W, Hq, Hkv, D, theta = 30, 8, 4, 2, 64, 1e6
    q, k, v, kraw, vc = _inputs(rng, L, W, Hq, Hkv, D)
    filled = np.array([1, 0, 1, 1, 0, 0, 1, 0], bool)

    def run(shift):
        kc = rope_rotate(kraw, (shift + np.arange(L))[:, None], theta)
        r = topological_reorder(filled, L)
        pos = r["pos"] + shift
        qp = rope_rotate(q[r["perm"]], pos[:, None], theta)
        kp = rope_rotate(k[r["perm"]], pos[:, None], theta)
        return window_attention_reordered(qp, kp, v[r["perm"]], kc, vc)

    base = run(0)
    for shift in (1, 1000, 31000):
        assert np.max(np.abs(run(shift) - base)) <= 1e-10
