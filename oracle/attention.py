"""Causal GQA window attention over [KV prefix ; window] (oracle; test infrastructure only).

hyper.ai summary of WeDLM, "Method": a causal forward pass over the reordered
window, conditioned on the persistent KV cache; the reordering lets every mask
see every observed token under a plain causal mask. sai.science review,
"Strengths": the causal mask itself is left untouched.

Two independent forms are given, so that one can be checked against the other:

  Form R (``window_attention_reordered``): the window is already in physical
    order (filled first); row p attends to all L prefix keys and to window rows
    0..p. This is the literal causal mask over physical order.

  Form M (``window_attention_masked``): the window stays in slot order; query
    slot i attends to all L prefix keys and to window slot j when
    ``visible_mask(filled)[i, j]`` holds. No reordering is done.

Readings: the diagonal is visible (a slot sees itself); mask slots see the
earlier mask slots in logical order; scale = 1/sqrt(D); query head h reads kv
head h // (Hq/Hkv); no soft-cap, ALiBi or sliding window; cached keys are
stored after RoPE.
"""

import numpy as np


def visible_mask(filled):
    """[W, W] bool: may query slot i see window slot j (slot order).

    A filled slot sees the filled slots at or before it; a mask slot sees every
    filled slot and the mask slots at or before it. This is what a causal mask
    over the physical order (filled ascending, then masks ascending) allows,
    written directly in slot terms.
    """
    f = np.asarray(filled, dtype=bool)
    W = f.shape[0]
    i = np.arange(W)[:, None]
    j = np.arange(W)[None, :]
    earlier_or_same = j <= i
    fi = f[:, None]
    fj = f[None, :]
    return (fj & (~fi | earlier_or_same)) | (~fi & ~fj & earlier_or_same)


def _attend(q, keys, values, allowed, scale):
    """softmax(scale * q keys^T, masked by allowed) @ values, float64.

    q [M, D], keys [N, D], values [N, D], allowed [M, N] bool (every row has at
    least one allowed key).
    """
    s = (q @ keys.T) * scale
    s = np.where(allowed, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    p = e / e.sum(axis=1, keepdims=True)
    return p @ values


def window_attention_reordered(q_phys, k_phys, v_phys, k_cache, v_cache, scale=None):
    """Form R: causal attention over [prefix ; window in physical order].

    Args (float arrays, promoted to float64):
      q_phys  [W, Hq, D]  rotated queries, physical order.
      k_phys  [W, Hkv, D] rotated keys, physical order.
      v_phys  [W, Hkv, D] values, physical order.
      k_cache [L, Hkv, D] rotated prefix keys (L may be 0).
      v_cache [L, Hkv, D] prefix values.
      scale   softmax scale, default 1/sqrt(D).

    Returns out_phys [W, Hq, D] float64.
    """
    q_phys = np.asarray(q_phys, np.float64)
    k_phys = np.asarray(k_phys, np.float64)
    v_phys = np.asarray(v_phys, np.float64)
    k_cache = np.asarray(k_cache, np.float64)
    v_cache = np.asarray(v_cache, np.float64)
    W, Hq, D = q_phys.shape
    Hkv = k_phys.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = Hq // Hkv
    L = k_cache.shape[0]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    # causal over physical order: row p sees prefix + window rows 0..p
    allowed = np.concatenate(
        [np.ones((W, L), dtype=bool), np.tril(np.ones((W, W), dtype=bool))], axis=1
    )
    out = np.empty((W, Hq, D), dtype=np.float64)
    for h in range(Hq):
        kv = h // g
        keys = np.concatenate([k_cache[:, kv, :], k_phys[:, kv, :]], axis=0)
        vals = np.concatenate([v_cache[:, kv, :], v_phys[:, kv, :]], axis=0)
        out[:, h, :] = _attend(q_phys[:, h, :], keys, vals, allowed, scale)
    return out


def window_attention_masked(q_slot, k_slot, v_slot, filled, k_cache, v_cache, scale=None):
    """Form M: the same attention in slot order with an explicit visibility mask.

    Args as in Form R but in slot order (q_slot/k_slot rotated at their logical
    positions), plus ``filled`` [W] bool. Returns out_slot [W, Hq, D].
    """
    q_slot = np.asarray(q_slot, np.float64)
    k_slot = np.asarray(k_slot, np.float64)
    v_slot = np.asarray(v_slot, np.float64)
    k_cache = np.asarray(k_cache, np.float64)
    v_cache = np.asarray(v_cache, np.float64)
    W, Hq, D = q_slot.shape
    Hkv = k_slot.shape[1]
    g = Hq // Hkv
    L = k_cache.shape[0]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    allowed = np.concatenate([np.ones((W, L), dtype=bool), visible_mask(filled)], axis=1)
    out = np.empty((W, Hq, D), dtype=np.float64)
    for h in range(Hq):
        kv = h // g
        keys = np.concatenate([k_cache[:, kv, :], k_slot[:, kv, :]], axis=0)
        vals = np.concatenate([v_cache[:, kv, :], v_slot[:, kv, :]], axis=0)
        out[:, h, :] = _attend(q_slot[:, h, :], keys, vals, allowed, scale)
    return out
