"""Decoding counters of a run of window steps: tokens and predictions per
forward, prefix cacheability and commit delay.

sai.science review of WeDLM, "Summary": the paper's efficiency argument is
prefix cacheability - how soon a proposed token enters the committed prefix
whose KV is never recomputed - measured by a p_cache that the review, under
"Strengths", calls under-specified. The definitions used here are this
project's:

  * tokens per forward      = committed tokens / (steps * sequences);
  * predictions per forward = slots filled by the selection / (steps * sequences);
  * commit delay of a token = the step that commits it minus the step whose
    selection filled it (1 at best: a slot filled in a step is committed in a
    later step, as a mask's KV in the forward cannot be kept);
  * p_cache                 = the fraction of committed tokens (filled during
    the run) whose delay is 1, i.e. that were cached by the very next forward.

These are measurements of a run, applied identically to the records of the
GPU path and of the oracle; they compute nothing of the method.
"""

import numpy as np


def decode_counters(records, W):
    """Counters of a run.

    Args:
      records: one dict per step, in order, with "prefix_len_in" [B] (the
        committed length before the step), "selected" [B, W] (slots the step
        filled) and "commit_len" [B] (tokens the step committed).
      W: window size.

    Returns dict: steps, sequences, committed, predicted, tokens_per_forward,
    predictions_per_forward, p_cache, mean_commit_delay, delay_histogram
    (delay -> count, for committed tokens filled during the run).
    """
    steps = len(records)
    if steps == 0:
        raise ValueError("no steps")
    B = len(records[0]["commit_len"])
    fill_step = [dict() for _ in range(B)]  # logical position -> step that filled it
    committed = 0
    predicted = 0
    delays = []
    for s, r in enumerate(records):
        L = np.asarray(r["prefix_len_in"], np.int64)
        sel = np.asarray(r["selected"], bool).reshape(B, W)
        c = np.asarray(r["commit_len"], np.int64)
        for b in range(B):
            # commits of this step: positions L .. L + c - 1, filled in earlier steps
            for p in range(int(L[b]), int(L[b] + c[b])):
                f = fill_step[b].pop(p, None)
                if f is not None:
                    delays.append(s - f)
            committed += int(c[b])
            for i in np.nonzero(sel[b])[0]:
                fill_step[b][int(L[b]) + int(i)] = s
                predicted += 1
    hist = {}
    for d in delays:
        hist[d] = hist.get(d, 0) + 1
    n = len(delays)
    return {
        "steps": steps,
        "sequences": B,
        "committed": committed,
        "predicted": predicted,
        "tokens_per_forward": committed / (steps * B),
        "predictions_per_forward": predicted / (steps * B),
        "p_cache": (hist.get(1, 0) / n) if n else None,
        "mean_commit_delay": (sum(delays) / n) if n else None,
        "delay_histogram": dict(sorted(hist.items())),
    }
