"""The oracle's pins fail on plausible mistakes (CPU).

Each test plants one mistake in a copy of an oracle function, swaps it into a
pin test's namespace and checks that the pin then fails. This shows that a
dropped term, a wrong sign, a wrong pairing or a wrong visibility rule in the
oracle would not go unnoticed.
"""

import numpy as np
import pytest

import oracle.rope as rope_mod
import tests.test_oracle_attention as t_attn
import tests.test_oracle_entropy as t_ent
import tests.test_oracle_rope as t_rope
import tests.test_oracle_select_commit as t_sel
from oracle import attention as attn_mod
from oracle import select as select_mod
from oracle.entropy import vocab_entropy_argmax as _orig_entropy


def _rope_sign_flipped(x, positions, theta):
    x = np.asarray(x, np.float64)
    half = x.shape[-1] // 2
    ang = np.asarray(positions, np.float64)[..., None] * rope_mod.rope_frequencies(x.shape[-1], theta)
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * c + hi * s, hi * c - lo * s], axis=-1)


def _rope_interleaved(x, positions, theta):
    x = np.asarray(x, np.float64)
    D = x.shape[-1]
    ang = np.asarray(positions, np.float64)[..., None] * rope_mod.rope_frequencies(D, theta)
    c, s = np.cos(ang), np.sin(ang)
    ev, od = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = ev * c - od * s
    y[..., 1::2] = od * c + ev * s
    return y


def test_rope_sign_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(t_rope, "rope_rotate", _rope_sign_flipped)
    with pytest.raises(AssertionError):
        t_rope.test_d2_is_complex_multiplication()


def test_rope_pairing_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(t_rope, "rope_rotate", _rope_interleaved)
    with pytest.raises(AssertionError):
        t_rope.test_rotate_half_pairing_closed_form()


def test_entropy_dropped_term_is_caught(monkeypatch):
    def no_t_term(logits):
        z = np.asarray(logits, np.float64)
        m = z.max(-1, keepdims=True)
        return np.log(np.exp(z - m).sum(-1)), np.argmax(z, -1)
    monkeypatch.setattr(t_ent, "vocab_entropy_argmax", no_t_term)
    with pytest.raises(AssertionError):
        t_ent.test_two_level_closed_form(512, 1, 8.0, 0.0)


def test_entropy_last_index_argmax_is_caught(monkeypatch):
    def last_argmax(logits):
        H, _ = _orig_entropy(logits)
        z = np.asarray(logits, np.float64)
        return H, z.shape[-1] - 1 - np.argmax(z[..., ::-1], -1)
    monkeypatch.setattr(t_ent, "vocab_entropy_argmax", last_argmax)
    with pytest.raises(AssertionError):
        t_ent.test_argmax_lowest_index_on_ties()


def test_visibility_mistake_is_caught(monkeypatch):
    def masks_see_only_earlier(filled):
        f = np.asarray(filled, bool)
        W = f.size
        return np.tril(np.ones((W, W), bool))          # plain slot-order causal mask
    monkeypatch.setattr(attn_mod, "visible_mask", masks_see_only_earlier)
    with pytest.raises(AssertionError):
        t_attn.test_form_r_equals_form_m_every_pattern_tiny_shape()


def test_missing_scale_is_caught(monkeypatch):
    orig = attn_mod.window_attention_reordered

    def unscaled(q, k, v, kc, vc, scale=None):
        return orig(q, k, v, kc, vc, scale=1.0)
    monkeypatch.setattr(t_attn, "window_attention_reordered", unscaled)
    with pytest.raises(AssertionError):
        t_attn.test_all_filled_window_is_ordinary_causal_attention(8, 8)


def test_penalty_sign_mistake_is_caught(monkeypatch):
    orig = select_mod.select_slots

    def minus_penalty(entropy, filled, lam, tau, min_fill=1, tie_eps=1e-4, adopt=None):
        return orig(entropy, filled, -lam, tau, min_fill, tie_eps, adopt)
    monkeypatch.setattr(t_sel, "select_slots", minus_penalty)
    case = next(c for c in t_sel.CASES if c["name"] == "distance_penalty_orders_slots")
    with pytest.raises(AssertionError):
        t_sel.test_golden_case(case)


def test_page_offset_mistake_is_caught(monkeypatch):
    import oracle.commit as commit_mod

    def wrong_slot(row, position, page_size):
        return int(row[position % len(row)]) * page_size + position % page_size
    monkeypatch.setattr(commit_mod, "cache_slot_of", wrong_slot)
    case = next(c for c in t_sel.CASES if c["name"] == "run_then_gap_commit_across_pages")
    with pytest.raises(AssertionError):
        t_sel.test_golden_case(case)


def test_projection_transposed_is_caught(monkeypatch):
    import tests.test_oracle_lm_head as t_lm

    def transposed(hidden, w_vocab):
        h = np.asarray(hidden, np.float64)
        w = np.asarray(w_vocab, np.float64)
        return h @ w[: h.shape[-1], : h.shape[-1]]  # rows taken for columns
    monkeypatch.setattr(t_lm, "vocab_projection", transposed)
    with pytest.raises((AssertionError, ValueError)):
        t_lm.test_one_hot_hidden_selects_a_column()


def test_projection_dropped_term_is_caught(monkeypatch):
    import tests.test_oracle_lm_head as t_lm

    def last_term_dropped(hidden, w_vocab):
        h = np.asarray(hidden, np.float64)[..., :-1]
        w = np.asarray(w_vocab, np.float64)[:, :-1]
        return h @ w.T
    monkeypatch.setattr(t_lm, "vocab_projection", last_term_dropped)
    with pytest.raises(AssertionError):
        t_lm.test_brute_force_small()


def test_dual_stream_own_block_memory_leak_is_caught(monkeypatch):
    import oracle.dual_stream as ds
    import tests.test_oracle_dual_stream as t_ds
    orig = ds.dual_stream_visibility

    def leaky(filled, block):
        vis = orig(filled, block)
        N = len(filled)
        for t in range(N):
            j0 = (t // block) * block
            vis[N + t, j0:min(j0 + block, N)] = True  # the clean copy of its own block
        return vis
    monkeypatch.setattr(ds, "dual_stream_visibility", leaky)
    with pytest.raises(AssertionError):
        t_ds.test_no_leakage()


def test_dual_stream_masks_first_is_caught(monkeypatch):
    import oracle.dual_stream as ds
    import tests.test_oracle_dual_stream as t_ds
    orig = ds.block_rank

    def masks_first(filled, block):
        return orig(~np.asarray(filled, bool), block)
    monkeypatch.setattr(ds, "block_rank", masks_first)
    with pytest.raises(AssertionError):
        t_ds.test_mask_form_equals_reordered_form()
