"""One window step and the streaming loop, composed from the oracle's parts (test infrastructure only).

hyper.ai summary of WeDLM, "Method" (Streaming Parallel Decoding): per step,
reorder the window (filled first, logical positions kept), run one causal
forward over it conditioned on the persistent KV cache, select the positions to
fill by distance-penalised entropy, commit the leftmost contiguous filled run
to the cache and append masks. "Key Contributions": a fixed parallel workload
per step. With synthetic inputs the forward's logits are inputs of the step;
several independent layers share one reorder and one commit length.
"""

import numpy as np

from .reorder import topological_reorder
from .rope import rope_rotate
from .attention import window_attention_reordered
from .entropy import vocab_entropy_argmax
from .select import select_slots
from .commit import commit_and_refill


def window_step(filled, tokens, prefix_len, q, k, v, k_cache, v_cache, logits, block_table,
                theta, lam, tau, page_size, min_fill=1, mask_id=-1, layers=None, scale=None,
                adopt_selected=None, store=None, commit_rule="stream", workers=1):
    """One window step for a batch of sequences and n_layers independent layers.

    Args:
      filled [B, W] bool, tokens [B, W] int, prefix_len [B] int: window state.
      q [n_layers, B, W, Hq, D], k, v [n_layers, B, W, Hkv, D]: window
        projections in slot order, before RoPE.
      k_cache, v_cache: k_cache[layer][b] is [L_b, Hkv, D] (keys already rotated),
        v_cache likewise. Only the layers in ``layers`` are read.
      logits [B, W, V]: slot order.
      block_table [B, max_pages]: page ids per sequence.
      layers: layer indices whose attention is computed (default: all).
      adopt_selected: optional callable(b) -> [W] bool, another
        implementation's selection for sequence b; only the flagged near-tie
        decisions take it (``select_slots``' ``adopt``).
      store: optional callable mapping a float64 array to the values a storage
        type holds (e.g. one round-to-nearest-even to bf16). When given, the
        rotated window rows are stored through it before they are attended to
        and committed: the rows a bf16 cache receives are bf16 values. The
        returned q_phys / k_phys / v_phys stay unrounded.
      commit_rule: "stream" (commit the leading filled run) or "block" (commit
        the window only once it is entirely filled); see ``commit_count``.
      workers: threads for the entropy's independent rows (same result).

    Returns a dict of float64 / int64 numpy results (see keys below).
    """
    filled = np.asarray(filled, dtype=bool)
    tokens = np.asarray(tokens, dtype=np.int64)
    prefix_len = np.asarray(prefix_len, dtype=np.int64)
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    n_layers, B, W, Hq, D = q.shape
    Hkv = k.shape[3]
    if layers is None:
        layers = range(n_layers)
    layers = list(layers)

    out = {
        "filled_in": filled.copy(), "tokens_in": tokens.copy(), "prefix_len_in": prefix_len.copy(),
        "perm": np.zeros((B, W), np.int64), "inv": np.zeros((B, W), np.int64),
        "pos": np.zeros((B, W), np.int64), "n_obs": np.zeros(B, np.int64),
        "run": np.zeros(B, np.int64),
    }
    for b in range(B):
        r = topological_reorder(filled[b], prefix_len[b])
        for key in ("perm", "inv", "pos"):
            out[key][b] = r[key]
        out["n_obs"][b] = r["n_obs"]
        out["run"][b] = r["run"]

    # RoPE at logical positions, gathered into physical order
    q_phys = np.empty((n_layers, B, W, Hq, D), np.float64)
    k_phys = np.empty((n_layers, B, W, Hkv, D), np.float64)
    v_phys = np.empty((n_layers, B, W, Hkv, D), np.float64)
    for b in range(B):
        perm = out["perm"][b]
        pos = out["pos"][b]
        q_phys[:, b] = rope_rotate(q[:, b][:, perm], pos[None, :, None], theta)
        k_phys[:, b] = rope_rotate(k[:, b][:, perm], pos[None, :, None], theta)
        v_phys[:, b] = np.asarray(v[:, b][:, perm], np.float64)
    out["q_phys"], out["k_phys"], out["v_phys"] = q_phys, k_phys, v_phys

    keep = store if store is not None else (lambda x: x)
    attn = {}
    for layer in layers:
        o = np.empty((B, W, Hq, D), np.float64)
        for b in range(B):
            o[b] = window_attention_reordered(keep(q_phys[layer, b]), keep(k_phys[layer, b]),
                                              keep(v_phys[layer, b]), k_cache[layer][b],
                                              v_cache[layer][b], scale)
        attn[layer] = o
    out["attn_out_phys"] = attn

    H, a = vocab_entropy_argmax(logits, workers=workers)
    out["entropy"], out["argmax"] = H, a
    out["score"] = np.zeros((B, W), np.float64)
    out["selected"] = np.zeros((B, W), bool)
    out["fallback"] = np.zeros(B, bool)
    out["flags"] = []
    for b in range(B):
        other = None if adopt_selected is None else adopt_selected(b)
        s = select_slots(H[b], filled[b], lam, tau, min_fill, adopt=other)
        out["flags"].extend((b, kind, i) for kind, i in s["flags"])
        out["score"][b] = s["score"]
        out["selected"][b] = s["selected"]
        out["fallback"][b] = s["fallback"]

    out["commit_len"] = np.zeros(B, np.int64)
    out["cache_slot"] = np.full((B, W), -1, np.int64)
    out["committed"] = []
    new_tokens = np.empty_like(tokens)
    new_filled = np.empty_like(filled)
    new_len = np.empty_like(prefix_len)
    for b in range(B):
        c = commit_and_refill(tokens[b], filled[b], prefix_len[b], out["run"][b], out["selected"][b],
                              a[b], block_table[b], page_size, mask_id, rule=commit_rule)
        out["commit_len"][b] = c["commit_len"]
        out["cache_slot"][b] = c["cache_slot"]
        out["committed"].append(c["committed"])
        new_tokens[b], new_filled[b], new_len[b] = c["tokens"], c["filled"], c["prefix_len"]
    out["tokens"], out["filled"], out["prefix_len"] = new_tokens, new_filled, new_len
    return out


class _Growable:
    """Append-only float64 row buffer (avoids re-copying a cache every step)."""

    def __init__(self, rows, capacity):
        rows = np.asarray(rows, np.float64)
        self.n = rows.shape[0]
        self.buf = np.empty((max(capacity, self.n),) + rows.shape[1:], np.float64)
        self.buf[: self.n] = rows

    def append(self, rows):
        m = rows.shape[0]
        if self.n + m > self.buf.shape[0]:
            grown = np.empty((2 * (self.n + m),) + self.buf.shape[1:], np.float64)
            grown[: self.n] = self.buf[: self.n]
            self.buf = grown
        self.buf[self.n: self.n + m] = rows
        self.n += m

    def view(self):
        return self.buf[: self.n]


def stream_loop(filled, tokens, prefix_len, k_cache, v_cache, block_table, steps, inputs_for_step,
                theta, lam, tau, page_size, min_fill=1, mask_id=-1, attend=None, track_layers=(),
                adopt_selected=None, on_step=None, store=None, commit_rule="stream", workers=1):
    """Run the streaming decoder for ``steps`` window steps.

    Args:
      filled, tokens, prefix_len, block_table: initial window state.
      k_cache, v_cache: initial caches, [layer][b] -> [L_b, Hkv, D] for every
        layer in ``track_layers`` (other layers' caches are not tracked).
      inputs_for_step(s) -> (q, k, v, logits) for step s, shapes as in
        ``window_step``.
      attend(s) -> layers whose attention to compute at step s (default none);
        they must be tracked layers.
      adopt_selected(s, b) -> [W] bool: another implementation's selection at
        step s, taken only by flagged near-tie decisions.
      on_step(s, result) is called after each step with window_step's result.
      store: as in ``window_step``; committed rows enter the tracked caches
        through it too.
      commit_rule: as in ``window_step`` ("block" gives the stop-and-wait
        decoder on the same steps).
      workers: as in ``window_step``.

    Returns dict with per-step commit lengths [steps, B], the final state and
    the total committed tokens.
    """
    filled = np.asarray(filled, bool).copy()
    tokens = np.asarray(tokens, np.int64).copy()
    prefix_len = np.asarray(prefix_len, np.int64).copy()
    track_layers = list(track_layers)
    caches = {}
    for layer in track_layers:
        caches[layer] = ([_Growable(k_cache[layer][b], len(k_cache[layer][b]) + 64)
                          for b in range(len(prefix_len))],
                         [_Growable(v_cache[layer][b], len(v_cache[layer][b]) + 64)
                          for b in range(len(prefix_len))])
    commit_log = []
    for s in range(steps):
        q, k, v, logits = inputs_for_step(s)
        layers = list(attend(s)) if attend is not None else []
        n_layers = np.asarray(q).shape[0]
        kc = [None] * n_layers
        vc = [None] * n_layers
        for layer in layers:
            kc[layer] = [g.view() for g in caches[layer][0]]
            vc[layer] = [g.view() for g in caches[layer][1]]
        ov = None
        if adopt_selected is not None:
            ov = (lambda b, _s=s: adopt_selected(_s, b))
        r = window_step(filled, tokens, prefix_len, q, k, v, kc, vc, logits, block_table, theta, lam,
                        tau, page_size, min_fill, mask_id, layers=layers, adopt_selected=ov,
                        store=store, commit_rule=commit_rule, workers=workers)
        keep = store if store is not None else (lambda x: x)
        for layer in track_layers:
            for b in range(len(prefix_len)):
                c = int(r["commit_len"][b])
                if c:
                    caches[layer][0][b].append(keep(r["k_phys"][layer, b, :c]))
                    caches[layer][1][b].append(keep(r["v_phys"][layer, b, :c]))
        commit_log.append(r["commit_len"].copy())
        if on_step is not None:
            on_step(s, r)
        filled, tokens, prefix_len = r["filled"], r["tokens"], r["prefix_len"]
    return {
        "commit_len": np.array(commit_log, np.int64).reshape(steps, -1),
        "filled": filled, "tokens": tokens, "prefix_len": prefix_len,
        "total_committed": int(np.sum(commit_log)) if commit_log else 0,
        "caches": {layer: ([g.view() for g in caches[layer][0]], [g.view() for g in caches[layer][1]])
                   for layer in track_layers},
    }
