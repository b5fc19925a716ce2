"""Full-vocabulary softmax entropy and argmax per slot (oracle; test infrastructure only).

hyper.ai summary of WeDLM, "Method": slots are chosen by a distance-penalised
entropy rule. sai.science review, "Weaknesses": the score is an entropy per
position adjusted by a distance term.

Readings: Shannon entropy in nats of the temperature-1 softmax over the whole
vocabulary; the token that fills a slot is the argmax of its logits, the lowest
vocabulary id among equal maxima (greedy decoding instead of the evaluation's
temperature sampling, which would need a shared random stream).
"""

from concurrent.futures import ThreadPoolExecutor

import numpy as np


def vocab_entropy_argmax(logits, workers=1):
    """Entropy (nats) and argmax of softmax(logits) along the last axis.

    Args:
      logits: float array [..., V] (promoted to float64; -inf entries allowed
              as long as every row has a finite maximum).
      workers: rows are independent; with workers > 1 they are dealt out in
              contiguous chunks to that many threads (each row's arithmetic is
              unchanged, so the result is the same bit for bit).

    Returns (entropy float64 [...], argmax int64 [...]):
      p = softmax(z), H = -sum_v p_v ln p_v (terms with p_v = 0 count 0),
      argmax = lowest v with z_v = max z.
    """
    z = np.asarray(logits)
    if workers > 1 and z.ndim > 1 and z.shape[-1] > 0:
        rows = z.reshape(-1, z.shape[-1])
        chunks = np.array_split(np.arange(rows.shape[0]), min(workers, rows.shape[0]))
        with ThreadPoolExecutor(len(chunks)) as pool:
            parts = list(pool.map(lambda c: _rows_entropy_argmax(rows[c[0]: c[-1] + 1]), chunks))
        H = np.concatenate([h for h, _ in parts]).reshape(z.shape[:-1])
        a = np.concatenate([x for _, x in parts]).reshape(z.shape[:-1])
        return H, a
    return _rows_entropy_argmax(z)


def _rows_entropy_argmax(logits):
    z = np.asarray(logits, dtype=np.float64)
    m = z.max(axis=-1, keepdims=True)
    shifted = z - m
    e = np.exp(shifted)
    s = e.sum(axis=-1, keepdims=True)
    p = e / s
    log_p = shifted - np.log(s)
    with np.errstate(invalid="ignore"):          # 0 * -inf where p underflows to 0
        terms = np.where(p > 0.0, p * log_p, 0.0)
    H = -terms.sum(axis=-1)
    # np.argmax returns the first occurrence of the maximum
    a = np.argmax(z, axis=-1).astype(np.int64)
    return H, a
