"""Fused vocabulary projection + entropy selection against the oracle (GPU).

The GPU computes the logits in fp32 from bf16 hidden states and projection
rows and never stores them; the oracle forms them in float64 from the same
stored values. Entropy |dH| <= 1e-3; argmax exact, except that a row whose
GPU argmax lies within 1e-4 of the oracle's largest logit is a flagged near
tie (counted and reported); score within the entropy bar (it is formed from
the GPU's entropy); selection exact on every slot, a decision the oracle flags
as a near tie (within 1e-4) taking the GPU's choice for that comparison only.
Shapes cover one, two and four 32-row blocks per workgroup, several row
groups, a ragged last vocabulary tile and packed block, one to many rotations
of the chunk loop and the full Qwen3-8B / Qwen2.5-7B projections (every
sequence). The packed layout is checked element by element against its
documented index formula.
"""

import numpy as np
import pytest
import torch

import oracle
from causal_streaming_decoding_amd import wedlm as W
from causal_streaming_decoding_amd.synth import lm_head_inputs, to_f64

from .parity import ENTROPY_ATOL

pytestmark = pytest.mark.gpu

LAM, TAU = 0.1, 1.0
TIE = 1e-4  # the near-tie band of the stated parity bar


def _pack(hidden, V, w):
    nbytes = W.wedlm_lm_head_packed_size(W.WEDLM_BF16, hidden, V)
    wp = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=w.device)
    W.wedlm_lm_head_pack(W.WEDLM_BF16, hidden, V, w, wp)
    return wp


def _gpu(B, Wn, hidden, V, h, w, filled, lam=LAM, tau=TAU, min_fill=1):
    dev = h.device
    wp = _pack(hidden, V, w)
    ent = torch.empty((B, Wn), dtype=torch.float32, device=dev)
    score = torch.empty_like(ent)
    arg = torch.empty((B, Wn), dtype=torch.int32, device=dev)
    sel = torch.empty((B, Wn), dtype=torch.uint8, device=dev)
    nbytes = W.wedlm_lm_head_select_workspace_size(W.WEDLM_BF16, B, Wn, hidden, V)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    W.wedlm_lm_head_select(W.WEDLM_BF16, B, Wn, hidden, V, h, wp, filled, lam, tau, min_fill, ent,
                           score, arg, sel, ws, nbytes)
    torch.cuda.synchronize()
    return {"entropy": ent.cpu().numpy(), "score": score.cpu().numpy(),
            "argmax": arg.cpu().numpy(), "selected": sel.cpu().numpy().astype(bool)}


def _oracle_rows(h64, w, seqs):
    """Oracle logits of the given sequences, the projection converted in slices."""
    V = w.shape[0]
    z = np.empty((len(seqs), h64.shape[1], V))
    step = 16384
    for v0 in range(0, V, step):
        wb = to_f64(w[v0:v0 + step])
        z[:, :, v0:v0 + step] = oracle.vocab_projection(h64[seqs], wb)
    return z


def _compare(gpu, h, w, filled, seqs, lam=LAM, tau=TAU, min_fill=1):
    h64 = to_f64(h)
    f = filled.cpu().numpy().astype(bool)
    z = _oracle_rows(h64, w, seqs)
    H, a = oracle.vocab_entropy_argmax(z, workers=8)
    near = 0
    flags = 0
    worst = 0.0
    for j, b in enumerate(seqs):
        dH = np.abs(gpu["entropy"][b] - H[j])
        assert (dH <= ENTROPY_ATOL).all(), ("entropy", b, float(dH.max()))
        for i in range(z.shape[1]):
            ga = int(gpu["argmax"][b, i])
            if ga != a[j, i]:
                # a flagged near tie: the GPU's token is within the band of the maximum
                assert 0 <= ga < z.shape[2], ("argmax", b, i, ga)
                assert z[j, i, ga] > z[j, i].max() - TIE, ("argmax", b, i, ga, int(a[j, i]))
                near += 1
        r = oracle.select_slots(H[j], f[b], lam, tau, min_fill, tie_eps=TIE,
                                adopt=gpu["selected"][b])
        flags += len(r["flags"])
        # the score carries the entropy's error; every decision must still agree
        dS = np.abs(gpu["score"][b].astype(np.float64) - r["score"])
        assert (dS <= ENTROPY_ATOL).all(), ("score", b, float(dS.max()))
        assert np.array_equal(gpu["selected"][b], r["selected"]), ("selected", b)
        worst = max(worst, float(dH.max()))
    print(f"[lm_head] {len(seqs)} sequences: max |dH| {worst:.2e}, argmax near ties (< {TIE}) "
          f"{near}, flagged selection decisions {flags}", flush=True)
    return near, flags


@pytest.mark.parametrize("B,Wn,hidden,V,spike", [
    (1, 16, 256, 5000, None),        # one 32-row block, ragged last vocabulary tile, one rotation
    (2, 32, 512, 4096, None),        # two blocks, exact tiles
    (3, 32, 256, 3001, (16.0, 20.0)),  # four blocks, low-entropy slots (threshold fires)
    (5, 40, 768, 2600, None),        # 200 rows: two row groups, the last ragged
    (1, 1, 256, 1, None),            # one slot, one vocabulary entry
    (4, 32, 1280, 2048, (6.0, 12.0)),  # five rotations of the chunk loop
    (2, 16, 1024, 700, None),        # a vocabulary smaller than three tiles
    (1, 5, 256, 33, None),           # a packed block that is mostly padding
    (3, 60, 512, 3000, None),        # 180 rows: eight 32-row blocks, the last ragged
    (6, 64, 256, 1000, (16.0, 20.0)),  # 384 rows: two workgroups of 256 and 128 rows
])
def test_lm_head_small(B, Wn, hidden, V, spike):
    print(f"[lm_head] B={B} W={Wn} hidden={hidden} V={V} spike={spike}", flush=True)
    h, w, filled = lm_head_inputs(B, Wn, hidden, V, "cuda", seed=B + V, spike=spike)
    gpu = _gpu(B, Wn, hidden, V, h, w, filled)
    _compare(gpu, h, w, filled, list(range(B)))
    if spike is not None and spike[0] >= 16.0:
        assert gpu["selected"].sum() > B  # the threshold fired beyond the one-per-sequence floor


@pytest.mark.parametrize("B,Wn,hidden,V", [
    (16, 16, 4096, 151936),   # Qwen3-8B projection, 256 rows
    (1, 16, 4096, 151936),    # one sequence, 16 rows
    (16, 32, 3584, 152064),   # Qwen2.5-7B projection, 512 rows
])
def test_lm_head_full_vocab(B, Wn, hidden, V):
    print(f"[lm_head] full B={B} W={Wn} hidden={hidden} V={V}", flush=True)
    h, w, filled = lm_head_inputs(B, Wn, hidden, V, "cuda", seed=7)
    gpu = _gpu(B, Wn, hidden, V, h, w, filled)
    assert np.isfinite(gpu["entropy"]).all()
    assert ((gpu["argmax"] >= 0) & (gpu["argmax"] < V)).all()
    # a sequence with a mask slot selects at least one slot (floor rule)
    f = filled.cpu().numpy().astype(bool)
    for b in range(B):
        assert gpu["selected"][b].any() == (~f[b]).any()
        assert not (gpu["selected"][b] & f[b]).any()
    # every sequence (float64 logits of all rows: up to ~620 MB on the host)
    _compare(gpu, h, w, filled, list(range(B)))


def test_lm_head_deterministic():
    B, Wn, hidden, V = 4, 32, 1024, 40000
    h, w, filled = lm_head_inputs(B, Wn, hidden, V, "cuda", seed=11)
    g1 = _gpu(B, Wn, hidden, V, h, w, filled)
    g2 = _gpu(B, Wn, hidden, V, h, w, filled)
    for k in g1:
        assert np.array_equal(g1[k], g2[k]), k


def test_lm_head_pack_layout():
    hidden, V = 512, 70  # three blocks, the last with 26 zero rows
    g = torch.Generator(device="cuda").manual_seed(3)
    w = torch.randn((V, hidden), generator=g, device="cuda").to(torch.bfloat16)
    wp = _pack(hidden, V, w).view(torch.int16).cpu().numpy()
    wr = w.view(torch.int16).cpu().numpy()
    nk = hidden // 64
    blocks = (V + 31) // 32
    assert wp.size == blocks * 32 * hidden
    for b in range(blocks):
        for c in range(nk):
            tile = wp[(b * nk + c) * 2048:(b * nk + c + 1) * 2048].reshape(4, 2, 32, 8)
            for ks in range(4):
                for kg in range(2):
                    for li in range(32):
                        v = 32 * b + li
                        k = 64 * c + 32 * kg + 8 * ks
                        expect = wr[v, k:k + 8] if v < V else np.zeros(8, np.int16)
                        assert np.array_equal(tile[ks, kg, li], expect), (b, c, ks, kg, li)
