"""Dual-stream masking attention (oracle; test infrastructure only).

hyper.ai summary of WeDLM, "Method": training pairs a clean memory stream
with a masked prediction stream over the same logical positions. The
prediction stream is cut into blocks, each topologically reordered (observed
tokens first, masks after, logical positions kept); a prediction token
attends to the clean memory-stream context of the preceding blocks and,
inside its own block, under the standard causal mask.

Readings (the pages give the rule only in words):
  * the memory stream attends causally to itself (causal LM attention);
  * a prediction token of block j = t // Bk sees every memory token at a
    position < j * Bk, and the prediction tokens of its own block that come
    before it in the block's physical order - observed tokens first, then
    masks, each group in ascending position - itself included; it sees no
    memory token of its own or a later block and no prediction token of
    another block;
  * RoPE rotates queries and keys of both streams at their logical
    positions (RoFormer, mlsanity.com page, "Builds on");
  * GQA: query head h reads kv head h // (Hq / Hkv); scale 1 / sqrt(D).

Written as an explicit visibility mask over the 2N keys [memory ; prediction]
followed by a masked softmax, in float64.
"""

import numpy as np

from .rope import rope_rotate


def block_rank(filled, block):
    """Physical index of every position inside its block: observed positions
    first, then masks, each in ascending order."""
    f = np.asarray(filled, bool)
    N = f.shape[0]
    rank = np.empty(N, np.int64)
    for b0 in range(0, N, block):
        fb = f[b0:b0 + block]
        n_obs = int(fb.sum())
        seen_obs = seen_msk = 0
        for i, obs in enumerate(fb):
            if obs:
                rank[b0 + i] = seen_obs
                seen_obs += 1
            else:
                rank[b0 + i] = n_obs + seen_msk
                seen_msk += 1
    return rank


def dual_stream_visibility(filled, block):
    """Boolean [2N, 2N]: row = query, column = key, both ordered
    [memory 0..N-1 ; prediction 0..N-1] by logical position."""
    f = np.asarray(filled, bool)
    N = f.shape[0]
    rank = block_rank(f, block)
    vis = np.zeros((2 * N, 2 * N), bool)
    for t in range(N):
        vis[t, :t + 1] = True                      # memory: causal over memory
        j0 = (t // block) * block
        vis[N + t, :j0] = True                     # earlier blocks' clean context
        for u in range(j0, min(j0 + block, N)):    # own block, physical causal
            if rank[u] <= rank[t]:
                vis[N + t, N + u] = True
    return vis


def dual_stream_attention(q_mem, k_mem, v_mem, q_pred, k_pred, v_pred, filled, block, theta,
                          scale=None, store=None):
    """Outputs of both streams, in logical (slot) order.

    Args:
      q_mem, q_pred: [N, Hq, D]; k_mem, v_mem, k_pred, v_pred: [N, Hkv, D]
        (before RoPE).
      filled: [N] bool, the prediction stream's observed positions.
      block: block size Bk.
      store: optional rounding of the rotated rows to a storage type, applied
        before the products (as a bf16 pipeline stores them).

    Returns (out_mem [N, Hq, D], out_pred [N, Hq, D]) float64.
    """
    keep = store if store is not None else (lambda x: x)
    q_mem, k_mem, v_mem = (np.asarray(x, np.float64) for x in (q_mem, k_mem, v_mem))
    q_pred, k_pred, v_pred = (np.asarray(x, np.float64) for x in (q_pred, k_pred, v_pred))
    N, Hq, D = q_mem.shape
    Hkv = k_mem.shape[1]
    g = Hq // Hkv
    scale = D ** -0.5 if scale is None else scale
    pos = np.arange(N)[:, None]
    q = np.concatenate([keep(rope_rotate(q_mem, pos, theta)), keep(rope_rotate(q_pred, pos, theta))])
    k = np.concatenate([keep(rope_rotate(k_mem, pos, theta)), keep(rope_rotate(k_pred, pos, theta))])
    v = np.concatenate([keep(v_mem), keep(v_pred)])
    vis = dual_stream_visibility(filled, block)
    out = np.empty((2 * N, Hq, D))
    for h in range(Hq):
        s = (q[:, h] @ k[:, h // g].T) * scale
        s = np.where(vis, s, -np.inf)
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, h] = p @ v[:, h // g]
    return out[:N], out[N:]
