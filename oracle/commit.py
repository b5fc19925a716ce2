"""Commit of the leftmost filled run, paged append and refill (oracle; test infrastructure only).

hyper.ai summary of WeDLM, "Method": the leftmost contiguous filled prefix of
the window is committed to the cache at once, because under the causal mask
its KV states depend only on earlier tokens; new mask tokens are appended so
the window keeps its size. mlsanity.com page, "Builds on": PagedAttention
(the cache is a pool of fixed-size pages addressed through a block table).

The same page's "Method" contrasts this with block decoding, where no token
of a block is cached before the whole block is finalised; the sai.science
review, "Reproducibility & code", notes that this block-wise baseline is not
in the released engine. ``commit_count`` gives both rules.

Readings:
  * the run is measured over the filled flags the forward pass saw; a slot
    filled by this step's selection is committed one step later at the
    earliest (its KV in this forward is the KV of a mask);
  * physical rows 0..c-1 are slots 0..c-1, so their rotated K and their V are
    appended at logical positions L .. L+c-1;
  * position t lives at flat cache slot block_table[t // P] * P + t % P;
  * the window shifts left by c; c masks (token id ``mask_id``) are appended;
    L grows by c.
"""

import numpy as np


def cache_slot_of(block_table_row, position, page_size):
    """Flat cache slot of a logical position: page id * P + offset in page."""
    return int(block_table_row[position // page_size]) * page_size + position % page_size


def commit_count(run, W, rule="stream"):
    """Tokens committed this step from the leading filled run.

    rule "stream": the whole leading run (streaming decoding);
    rule "block": the whole window once every slot is filled, else nothing
    (block-wise, stop-and-wait decoding: the window is one block that is
    cached only when finalised, then replaced by W masks).
    """
    if rule == "stream":
        return int(run)
    if rule == "block":
        return int(W) if int(run) == int(W) else 0
    raise ValueError(f"unknown commit rule {rule!r}")


def commit_and_refill(tokens, filled, prefix_len, run, selected, argmax_tok, block_table_row,
                      page_size, mask_id=-1, rule="stream"):
    """Commit one sequence's leading run (or block) and refill its window.

    Args:
      tokens, filled: [W] window state at forward time (slot order).
      prefix_len: L.
      run: leading filled run at forward time.
      selected, argmax_tok: [W] this step's fills.
      block_table_row: page ids of the sequence.
      rule: "stream" or "block" (see ``commit_count``).

    Returns dict: commit_len c, committed (token ids of slots 0..c-1),
    cache_slot [W] int64 (-1 past c), tokens, filled (new window), prefix_len.
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    f = np.asarray(filled, dtype=bool)
    sel = np.asarray(selected, dtype=bool)
    a = np.asarray(argmax_tok, dtype=np.int64)
    W = tokens.shape[0]
    L = int(prefix_len)
    r = int(run)
    if not (0 <= r <= W) or not f[:r].all() or (r < W and f[r]):
        raise ValueError("run is not the leading filled run of the window")
    c = commit_count(r, W, rule)

    cache_slot = np.full(W, -1, dtype=np.int64)
    for j in range(c):
        cache_slot[j] = cache_slot_of(block_table_row, L + j, page_size)
    committed = tokens[:c].copy()

    f_after = f | sel
    tok_after = np.where(sel, a, tokens)
    new_filled = np.concatenate([f_after[c:], np.zeros(c, dtype=bool)])
    new_tokens = np.concatenate([tok_after[c:], np.full(c, mask_id, dtype=np.int64)])
    return {
        "commit_len": c,
        "committed": committed,
        "cache_slot": cache_slot,
        "tokens": new_tokens,
        "filled": new_filled,
        "prefix_len": L + c,
    }
