"""Seeded synthetic inputs for the window step.

This module only draws random numbers and lays them out in plain logical
(per-sequence, slot-ordered) arrays. It holds none of the method's arithmetic:
no reordering, rotation, attention, entropy, selection or commit. Both the HIP
path (through ``layout.py``) and the CPU oracle consume what it returns.

Recipe (host side, ``numpy.random.default_rng(seed)`` = PCG64), draws in this
fixed order:
  1. prefix length of each sequence (fixed, uniform integers in [lo, hi], or
     an explicit list);
  2. a random permutation of the page pool, dealt out to the sequences in
     order, each getting enough pages for its prefix plus ``W * steps``
     positions (every step commits at most W tokens);
  3. prefix keys (already rotated) then prefix values, N(0, 1), per layer, per
     sequence: [L_b, Hkv, D];
  4. window q [n_layers, B, W, Hq, D], then k and v [n_layers, B, W, Hkv, D],
     N(0, 1), slot order, before RoPE;
  5. per sequence: how many slots are filled, which ones (without
     replacement), and a uniform token id for each filled slot;
  6. logits [B, W, V] ~ N(0, sigma^2) in float32, then the spikes (slot, token,
     magnitude) added in float32.
Every float tensor is then rounded once to the workload's storage type (bf16
by round-to-nearest-even); the returned float32 arrays hold exactly the stored
values, so both sides read identical numbers.

The streaming loop's per-step inputs are drawn on the device with torch's
generator (seeded with seed + step for the logits and an offset seed for the
window projections), because hundreds of steps of 36-layer inputs are too
large to draw on the host; the oracle reads host copies of the same tensors.
"""

import math

import numpy as np
import torch

from .workloads import Workload

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(wl: Workload):
    return _TORCH_DTYPE[wl.dtype]


def round_to_storage(x, dtype):
    """Round float32 numpy values to the storage type; returns float32 numpy."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    return torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()


def _prefix_lengths(wl, rng):
    kind = wl.prefix[0]
    if kind == "fixed":
        return np.full(wl.B, int(wl.prefix[1]), dtype=np.int64)
    if kind == "uniform":
        return rng.integers(wl.prefix[1], wl.prefix[2] + 1, size=wl.B).astype(np.int64)
    if kind == "list":  # explicit per-sequence lengths (no draw)
        lengths = np.asarray(wl.prefix[1], dtype=np.int64)
        if lengths.shape != (wl.B,):
            raise ValueError("prefix list needs one length per sequence")
        return lengths
    raise ValueError(kind)


def _page_pool(wl, lengths, steps, rng):
    P = wl.page_size
    need = [math.ceil((int(L) + wl.W * steps) / P) for L in lengths]
    num_pages = int(sum(need))
    pool = rng.permutation(num_pages).astype(np.int32)
    max_pages = max(need)
    table = np.zeros((wl.B, max_pages), dtype=np.int32)
    at = 0
    for b, n in enumerate(need):
        table[b, :n] = pool[at: at + n]
        # unused tail entries repeat the sequence's last page (never addressed)
        table[b, n:] = pool[at + n - 1]
        at += n
    return table, num_pages


def _filled(wl, rng):
    filled = np.zeros((wl.B, wl.W), dtype=bool)
    tokens = np.full((wl.B, wl.W), wl.mask_id, dtype=np.int64)
    kind = wl.fill[0]
    for b in range(wl.B):
        if kind == "none":
            n = 0
        elif kind == "count":
            n = int(wl.fill[1])
        elif kind in ("frac", "frac_per_seq"):
            n = int(round(rng.uniform(wl.fill[1], wl.fill[2]) * wl.W))
        else:
            raise ValueError(kind)
        slots = rng.choice(wl.W, size=n, replace=False)
        filled[b, slots] = True
        tokens[b, slots] = rng.integers(0, wl.V, size=n)
    return filled, tokens


def _spikes(wl, rng, rows):
    """List of (row, token, magnitude) for ``rows`` = B*W logit rows."""
    kind = wl.spike[0]
    out = []
    if kind == "none":
        return out
    if kind == "slots":
        n, mag = int(wl.spike[1]), float(wl.spike[2])
        for b in range(rows // wl.W):
            for s in rng.choice(wl.W, size=n, replace=False):
                out.append((b * wl.W + int(s), int(rng.integers(0, wl.V)), mag))
        return out
    if kind == "all_uniform":
        lo, hi = wl.spike[1], wl.spike[2]
        toks = rng.integers(0, wl.V, size=rows)
        mags = rng.uniform(lo, hi, size=rows)
        return [(r, int(toks[r]), float(mags[r])) for r in range(rows)]
    if kind == "prob":
        p, lo, hi = wl.spike[1], wl.spike[2], wl.spike[3]
        hit = rng.random(rows) < p
        toks = rng.integers(0, wl.V, size=rows)
        mags = rng.uniform(lo, hi, size=rows)
        return [(r, int(toks[r]), float(mags[r])) for r in range(rows) if hit[r]]
    raise ValueError(kind)


def make_step_inputs(wl: Workload, seed=None, steps=None, layers=None):
    """Inputs of one window step in logical layout (float32 numpy holding stored values).

    ``layers`` limits which layers' prefix caches are drawn (all by default);
    the window tensors always cover every layer. ``steps`` sets how many
    commits the page reservation must absorb (default: the workload's steps).

    Returns dict: prefix_len [B] int64, block_table [B, max_pages] int32,
    num_pages, k_cache/v_cache [layer][b] -> [L_b, Hkv, D] (None for layers not
    drawn), q [nl, B, W, Hq, D], k, v [nl, B, W, Hkv, D], filled [B, W] bool,
    tokens [B, W] int64, logits [B, W, V].
    """
    seed = wl.seed if seed is None else seed
    steps = wl.steps if steps is None else steps
    rng = np.random.default_rng(seed)
    lengths = _prefix_lengths(wl, rng)
    table, num_pages = _page_pool(wl, lengths, steps, rng)
    layers = range(wl.n_layers) if layers is None else list(layers)
    k_cache = [None] * wl.n_layers
    v_cache = [None] * wl.n_layers
    for layer in layers:
        k_cache[layer] = [round_to_storage(rng.standard_normal((int(L), wl.Hkv, wl.D), dtype=np.float32),
                                           wl.dtype) for L in lengths]
        v_cache[layer] = [round_to_storage(rng.standard_normal((int(L), wl.Hkv, wl.D), dtype=np.float32),
                                           wl.dtype) for L in lengths]
    nl = wl.n_layers
    q = round_to_storage(rng.standard_normal((nl, wl.B, wl.W, wl.Hq, wl.D), dtype=np.float32), wl.dtype)
    k = round_to_storage(rng.standard_normal((nl, wl.B, wl.W, wl.Hkv, wl.D), dtype=np.float32), wl.dtype)
    v = round_to_storage(rng.standard_normal((nl, wl.B, wl.W, wl.Hkv, wl.D), dtype=np.float32), wl.dtype)
    filled, tokens = _filled(wl, rng)
    rows = wl.B * wl.W
    logits = rng.standard_normal((rows, wl.V), dtype=np.float32) * np.float32(wl.logit_sigma)
    for r, tok, mag in _spikes(wl, rng, rows):
        logits[r, tok] += np.float32(mag)
    logits = round_to_storage(logits, wl.dtype).reshape(wl.B, wl.W, wl.V)
    return {
        "prefix_len": lengths, "block_table": table, "num_pages": num_pages,
        "k_cache": k_cache, "v_cache": v_cache, "q": q, "k": k, "v": v,
        "filled": filled, "tokens": tokens, "logits": logits,
    }


def stream_step_inputs(wl: Workload, step: int, device, seed=None):
    """Window q/k/v and logits of streaming step ``step``, drawn on ``device``.

    Logits: generator seeded with seed + step; N(0, sigma^2) float32, then
    every slot independently gets, with the spike probability, +U[lo, hi] on a
    uniform token; rounded once to the storage type. Window q, k, v: a second
    generator seeded with seed + step + 2**31, N(0, 1), rounded once.

    Returns (q, k, v, logits) torch tensors of the storage dtype on ``device``:
    q [nl, B, W, Hq, D], k/v [nl, B, W, Hkv, D], logits [B, W, V].
    """
    seed = wl.seed if seed is None else seed
    dt = torch_dtype(wl)
    rows = wl.B * wl.W
    g = torch.Generator(device=device)
    g.manual_seed(seed + step)
    z = torch.randn((rows, wl.V), generator=g, device=device, dtype=torch.float32)
    z.mul_(wl.logit_sigma)
    kind = wl.spike[0]
    if kind != "none":
        if kind == "prob":
            p, lo, hi = wl.spike[1], wl.spike[2], wl.spike[3]
        elif kind == "all_uniform":
            p, lo, hi = 1.0, wl.spike[1], wl.spike[2]
        else:
            raise ValueError("streaming inputs support probabilistic or per-slot spikes")
        hit = torch.rand(rows, generator=g, device=device) < p
        tok = torch.randint(0, wl.V, (rows,), generator=g, device=device)
        mag = torch.rand(rows, generator=g, device=device) * (hi - lo) + lo
        r = torch.arange(rows, device=device)
        z[r, tok] += torch.where(hit, mag, torch.zeros_like(mag))
    logits = z.to(dt).reshape(wl.B, wl.W, wl.V)
    g2 = torch.Generator(device=device)
    g2.manual_seed(seed + step + 2 ** 31)
    nl = wl.n_layers
    q = torch.randn((nl, wl.B, wl.W, wl.Hq, wl.D), generator=g2, device=device).to(dt)
    k = torch.randn((nl, wl.B, wl.W, wl.Hkv, wl.D), generator=g2, device=device).to(dt)
    v = torch.randn((nl, wl.B, wl.W, wl.Hkv, wl.D), generator=g2, device=device).to(dt)
    return q, k, v, logits


def lm_head_inputs(B, W, hidden, V, device, seed=0, logit_sigma=2.0, spike=None):
    """Inputs of the fused vocabulary projection + selection, drawn on ``device``.

    One torch generator seeded with ``seed``, draws in this order: hidden
    states [B, W, hidden] ~ N(0, 1); projection rows [V, hidden] ~
    N(0, logit_sigma^2 / hidden), so that the logits have standard deviation
    about ``logit_sigma`` like the logits workloads; filled flags [B, W], each
    slot with probability 1/2; then, when ``spike = (lo, hi)``, for every slot a
    uniform token t and a magnitude c ~ U[lo, hi], and the hidden state gets
    (c / logit_sigma^2) times row t of the projection added (its logit then
    rises by about c). Both float tensors are rounded once to bf16.

    Returns (hidden bf16 [B, W, hidden], w_vocab bf16 [V, hidden], filled uint8 [B, W]).
    """
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    h = torch.randn((B, W, hidden), generator=g, device=device, dtype=torch.float32)
    w = torch.randn((V, hidden), generator=g, device=device, dtype=torch.float32)
    w.mul_(logit_sigma / hidden ** 0.5)
    filled = (torch.rand((B, W), generator=g, device=device) < 0.5).to(torch.uint8)
    if spike is not None:
        lo, hi = spike
        tok = torch.randint(0, V, (B * W,), generator=g, device=device)
        mag = torch.rand(B * W, generator=g, device=device) * (hi - lo) + lo
        w_b = w.to(torch.bfloat16).to(torch.float32)  # the stored rows
        h.view(B * W, hidden).add_(w_b[tok] * (mag / logit_sigma ** 2)[:, None])
    return h.to(torch.bfloat16), w.to(torch.bfloat16), filled


def to_f64(t):
    """Host float64 copy of a torch tensor or numpy array (exact for f32/bf16)."""
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)
