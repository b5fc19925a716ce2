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
  * the fill decision is taken in float32 arithmetic: the kernel's precision,
    as the pages name none. The float64 margins are reported as flags when a
    decision is within ``tie_eps`` of flipping.
"""

import numpy as np


def select_slots(entropy, filled, lam, tau, min_fill=1, tie_eps=1e-4):
    """Choose the mask slots to fill in one window.

    Args:
      entropy: [W] per-slot entropy (nats).
      filled:  [W] bool, filled at forward time.
      lam, tau: penalty weight and threshold.
      min_fill: 1 to fill the lowest-score mask slot when none clears tau.
      tie_eps: margin under which a decision is flagged as a near tie.

    Returns dict:
      score     [W] float32  (H + lam * i, float32 arithmetic),
      selected  [W] bool,
      fallback  bool, the floor rule decided the step,
      flags     list of (kind, slot) near-tie flags.
    """
    H = np.asarray(entropy, dtype=np.float64)
    f = np.asarray(filled, dtype=bool)
    W = H.shape[0]
    lam32 = np.float32(lam)
    tau32 = np.float32(tau)
    idx32 = np.arange(W, dtype=np.float32)
    # two separate float32 roundings: the product, then the sum
    score = (H.astype(np.float32) + (lam32 * idx32).astype(np.float32)).astype(np.float32)
    score64 = H + float(lam) * np.arange(W, dtype=np.float64)

    candidates = [i for i in range(W) if not f[i]]
    selected = np.zeros(W, dtype=bool)
    flags = []
    for i in candidates:
        if score[i] < tau32:
            selected[i] = True
        if abs(score64[i] - float(tau)) < tie_eps:
            flags.append(("threshold", i))
    fallback = False
    if not selected.any() and candidates and min_fill == 1:
        best = min(candidates, key=lambda i: (score[i], i))
        selected[best] = True
        fallback = True
        for i in candidates:
            if i != best and abs(score64[i] - score64[best]) < tie_eps:
                flags.append(("fallback", i))
    return {"score": score, "selected": selected, "fallback": fallback, "flags": flags}
