"""Argmax ties and placement of the maximum in the entropy chunk pass (GPU).

The chunk pass keeps, per thread, only the start of the lowest 16-byte vector
holding its maximum and finds the element inside that one vector after the
block's reduction; the merges keep the lower index on equal maxima. These
cases put equal maxima where each of those steps decides: inside one vector,
in two vectors of one thread, in neighbouring threads, in two waves, in two
chunks, in the partial last chunk and at the row's last element, plus rows
whose every logit is equal. argmax must be the lowest index holding the
maximum (bit-exact against numpy's first occurrence); entropy within the
stated 1e-3 of the float64 oracle. Both the 16-byte vector path (V a multiple
of the vector width) and the single-element path, bf16 and fp32 logits.
"""

import numpy as np
import pytest
import torch

import oracle
from causal_streaming_decoding_amd import wedlm as W

from .parity import ENTROPY_ATOL

pytestmark = pytest.mark.gpu

CHUNK_BF16 = 256 * 8 * 8   # elements per chunk block: 256 threads x 8 vectors x 8 bf16
VEC_BF16 = 8


def _placements(V, vec, chunk):
    """Lists of indices that receive the row's maximum (all in range)."""
    out = [
        [0, V - 1],                          # first and last element
        [V - 1],                             # only the last (partial last chunk)
        [3, 5] if V > 5 else [0],            # one vector, two elements
        [vec - 1, vec] if V > vec else [0],  # the last of one vector, the first of the next thread's
        [7 + 256 * vec, 2 + 512 * vec] if V > 512 * vec + 2 else [V // 2],  # one thread, two vectors
        [64 * vec + 1, 1] if V > 64 * vec + 1 else [1 % V],                  # two waves
    ]
    if V > chunk + 5:
        out.append([chunk + 4, chunk - 1])   # last element of chunk 0, one of chunk 1
        out.append([V - 2, chunk + 5])       # chunk 1 and the last chunk
    return out


def _rows(V, vec, chunk, gen):
    rows = []
    for idx in _placements(V, vec, chunk):
        z = torch.randn(V, generator=gen) * 2.0
        z[idx] = 30.0                        # the maximum, exactly representable in bf16
        rows.append(z)
    rows.append(torch.zeros(V))              # every logit equal: argmax 0, H = ln V
    rows.append(torch.full((V,), -7.25))
    z = torch.full((V,), -3.0)
    z[-min(V, 3):] = 5.0                     # a run of maxima at the end
    rows.append(z)
    return torch.stack(rows)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("V", [151936, 152064, 16392, 16385, 1000, 8, 1])
def test_argmax_lowest_index_and_entropy(V, dtype):
    gen = torch.Generator().manual_seed(V)
    esize = 2 if dtype == torch.bfloat16 else 4
    vec = 16 // esize
    chunk = 256 * 8 * vec
    z = _rows(V, vec, chunk, gen).to(dtype)
    Wn = z.shape[0]
    zf = z.float().numpy().astype(np.float64)
    Href, aref = oracle.vocab_entropy_argmax(zf)
    dev = "cuda"
    zd = z.reshape(1, Wn, V).to(dev)
    dt = W.WEDLM_BF16 if dtype == torch.bfloat16 else W.WEDLM_F32
    filled = torch.zeros((1, Wn), dtype=torch.uint8, device=dev)
    ent = torch.empty((1, Wn), device=dev)
    sc = torch.empty_like(ent)
    am = torch.full((1, Wn), -5, dtype=torch.int32, device=dev)
    sel = torch.empty((1, Wn), dtype=torch.uint8, device=dev)
    nb = W.wedlm_entropy_select_workspace_size(dt, 1, Wn, V)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    W.wedlm_entropy_select(dt, 1, Wn, V, zd, filled, 0.0, 1.0, 1, ent, sc, am, sel, ws, nb)
    torch.cuda.synchronize()
    ga = am.cpu().numpy()[0].astype(np.int64)
    assert np.array_equal(ga, aref), (V, dtype, ga.tolist(), aref.tolist())
    dH = np.abs(ent.cpu().numpy()[0].astype(np.float64) - Href)
    assert (dH <= ENTROPY_ATOL).all(), (V, dtype, float(dH.max()))
    # the rows of equal logits: H = ln V exactly in the oracle
    assert abs(Href[-3] - np.log(V)) < 1e-9
