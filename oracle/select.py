"""Distance-penalised entropy selection of mask slots (oracle; test infrastructure only).

hyper.ai summary of WeDLM, "Method": a distance-penalised entropy rule picks
which positions to predict, favouring earlier positions so the committed
prefix grows left to right. sai.science review, "Weaknesses": the equation of
the adjusted entropy is missing from the text and its sign is open;
"Reproducibility & code": an entropy threshold flag controls filling, and
setting it to None gives one-by-one decoding; "Weaknesses": the quality tables
decode one token per step at the lowest-entropy position.

Readings (none of this is printed on the pages):
  * score_i = H_i + lambda * i, with i the 0-based distance of slot i from the
    window start (a penalty that grows with distance);
  * only mask slots are candidates; filled slots are never re-masked;
  * a candidate is filled when score_i < tau (strict);
  * if no candidate clears tau and min_fill is 1, the single candidate with
    the lowest score is filled (lowest slot on equal scores). PARITY UNPINNED:
    the pages never state what a step does when nothing clears the threshold;
    this is the one-token rule of their one-by-one mode applied as a floor.
  * every score and decision is float64, the definition itself. A decision
    whose float64 margin is under ``tie_eps`` is reported as a flag: another
    implementation that rounds differently may take it the other way.
"""

import numpy as np


def select_slots(entropy, filled, lam, tau, min_fill=1, tie_eps=1e-4, adopt=None):
    """Choose the mask slots to fill in one window.

    Args:
      entropy: [W] per-slot entropy (nats).
      filled:  [W] bool, filled at forward time.
      lam, tau: penalty weight and threshold.
      min_fill: 1 to fill the lowest-score mask slot when none clears tau.
      tie_eps: margin under which a decision is flagged as a near tie.
      adopt: optional [W] bool, another implementation's selection for this
        window. Only flagged decisions take it: a threshold comparison of
        slot i within tie_eps of tau takes adopt[i]; when the floor rule's
        lowest score has runners-up within tie_eps, the floor slot is the one
        of those tied candidates that adopt selects (when it selects exactly
        one). Every other decision is the oracle's own, so a caller comparing
        the two selections slot by slot still sees any unflagged difference.

    Returns dict:
      score     [W] float64 (H + lam * i),
      selected  [W] bool,
      fallback  bool, the floor rule decided the step,
      flags     list of (kind, slot) near-tie flags.
    """
    H = np.asarray(entropy, dtype=np.float64)
    f = np.asarray(filled, dtype=bool)
    W = H.shape[0]
    score = H + float(lam) * np.arange(W, dtype=np.float64)
    adopt = None if adopt is None else np.asarray(adopt, dtype=bool)

    candidates = [i for i in range(W) if not f[i]]
    selected = np.zeros(W, dtype=bool)
    flags = []
    for i in candidates:
        take = bool(score[i] < tau)
        if abs(score[i] - float(tau)) < tie_eps:
            flags.append(("threshold", i))
            if adopt is not None:
                take = bool(adopt[i])
        selected[i] = take
    fallback = False
    if not selected.any() and candidates and min_fill == 1:
        best = min(candidates, key=lambda i: (score[i], i))
        tied = [i for i in candidates if i != best and abs(score[i] - score[best]) < tie_eps]
        flags.extend(("fallback", i) for i in tied)
        if tied and adopt is not None:
            chosen = [i for i in [best] + tied if adopt[i]]
            if len(chosen) == 1:
                best = chosen[0]
        selected[best] = True
        fallback = True
    return {"score": score, "selected": selected, "fallback": fallback, "flags": flags}
