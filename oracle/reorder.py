"""Topological reordering of one window (oracle; test infrastructure only).

hyper.ai summary of WeDLM, "Method": observed (filled) tokens are moved to the
physical front, mask tokens to the end, and each token keeps its logical
position ID; in the streaming decoder this is done to the sliding window at
every step. sai.science review, "Summary": observed tokens are shifted to the
prefix while RoPE preserves logical positions.

Readings (the pages do not fix them):
  * the order inside the filled group and inside the mask group is the
    ascending logical order (a stable partition);
  * the window starts at the committed length L, so slot i has logical
    position L + i;
  * ``run`` is the length of the leading all-filled run of the window, used by
    the commit rule (leftmost contiguous filled prefix).
"""

import numpy as np


def topological_reorder(filled, prefix_len):
    """Reorder one window.

    Args:
      filled: sequence of W booleans, slot order (True = filled/observed).
      prefix_len: committed length L of the sequence.

    Returns a dict of int64 arrays / ints:
      perm[p]  slot held at physical index p,
      inv[i]   physical index of slot i,
      pos[p]   logical position of physical row p (= L + perm[p]),
      n_obs    number of filled slots,
      run      length of the leading filled run.
    """
    filled = [bool(f) for f in filled]
    W = len(filled)
    observed = [i for i in range(W) if filled[i]]
    masks = [i for i in range(W) if not filled[i]]
    perm = observed + masks
    inv = [0] * W
    for p, slot in enumerate(perm):
        inv[slot] = p
    pos = [int(prefix_len) + slot for slot in perm]
    run = 0
    while run < W and filled[run]:
        run += 1
    return {
        "perm": np.array(perm, dtype=np.int64),
        "inv": np.array(inv, dtype=np.int64),
        "pos": np.array(pos, dtype=np.int64),
        "n_obs": len(observed),
        "run": run,
    }
