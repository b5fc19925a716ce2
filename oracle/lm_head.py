"""Vocabulary projection followed by entropy selection (oracle; test infrastructure only).

hyper.ai summary of WeDLM, "Method": one causal forward pass over the window
yields the predictions that the distance-penalised entropy rule ranks. The
pass ends in the projection of each slot's final hidden state onto the
vocabulary.

Reading: that projection is a plain linear map, z_v = sum_k h_k W[v, k] (no
bias, no soft cap, no temperature); the entropy, argmax and selection that
follow are those of ``vocab_entropy_argmax`` and ``select_slots``.
"""

import numpy as np

from .entropy import vocab_entropy_argmax
from .select import select_slots


def vocab_projection(hidden, w_vocab):
    """Logits z[..., v] = sum_k hidden[..., k] * w_vocab[v, k], in float64.

    Args:
      hidden:  [..., hidden] final hidden states (promoted to float64).
      w_vocab: [V, hidden] projection, row v belongs to vocabulary entry v.
    """
    h = np.asarray(hidden, dtype=np.float64)
    w = np.asarray(w_vocab, dtype=np.float64)
    return h @ w.T


def lm_head_select(hidden, w_vocab, filled, lam, tau, min_fill=1, adopt=None):
    """Entropy, argmax and selection of every slot from its hidden state.

    Args:
      hidden:  [B, W, hidden]; w_vocab: [V, hidden]; filled: [B, W] bool.
      adopt: optional [B, W] bool, another implementation's selections, taken
        only by flagged near-tie decisions (``select_slots``).

    Returns dict: entropy [B, W] float64, argmax [B, W] int64, logits
    [B, W, V] float64, and per sequence the ``select_slots`` result
    (``select``: list of dicts).
    """
    z = vocab_projection(hidden, w_vocab)
    H, a = vocab_entropy_argmax(z)
    f = np.asarray(filled, dtype=bool)
    sel = [select_slots(H[b], f[b], lam, tau, min_fill,
                        adopt=None if adopt is None else adopt[b]) for b in range(H.shape[0])]
    return {"entropy": H, "argmax": a, "logits": z, "select": sel}
