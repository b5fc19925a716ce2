"""Workspace-free entropy selection against the workspace form, through the C ABI (GPU).

wedlm_entropy_select_noalloc runs the kernels of wedlm_entropy_select with
the chunk partials in the library's fixed device scratch instead of a caller
workspace; on the same inputs every output must be bitwise the same. Two calls
in a row, the second smaller than the first (the scratch then still holds the
first call's partials beyond the second's), then a third on logits whose rows
are not 16-byte aligned (the element-wise path). The smaller call is also held
to the oracle's bar (entropy within 1e-3, argmax and selection exact, a
flagged near tie taking the GPU's decision).
"""

import numpy as np
import pytest
import torch

import oracle
from causal_streaming_decoding_amd import wedlm as W

pytestmark = pytest.mark.gpu


def _inputs(B, Wn, V, seed, spike):
    g = torch.Generator(device="cuda").manual_seed(seed)
    z = torch.randn((B * Wn, V), generator=g, device="cuda") * 2.0
    tok = torch.randint(0, V, (B * Wn,), generator=g, device="cuda")
    mag = torch.rand(B * Wn, generator=g, device="cuda") * (spike[1] - spike[0]) + spike[0]
    z[torch.arange(B * Wn, device="cuda"), tok] += mag
    filled = (torch.rand((B, Wn), generator=g, device="cuda") < 0.5).to(torch.uint8)
    return z.to(torch.bfloat16).reshape(B, Wn, V), filled


def _outputs(B, Wn):
    # sentinels, so that an output the call does not write shows up
    return {"entropy": torch.full((B, Wn), float("nan"), device="cuda"),
            "score": torch.full((B, Wn), float("nan"), device="cuda"),
            "argmax": torch.full((B, Wn), -7, dtype=torch.int32, device="cuda"),
            "selected": torch.full((B, Wn), 7, dtype=torch.uint8, device="cuda")}


def _workspace_form(B, Wn, V, z, filled, lam, tau, min_fill):
    o = _outputs(B, Wn)
    nbytes = W.wedlm_entropy_select_workspace_size(W.WEDLM_BF16, B, Wn, V)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    W.wedlm_entropy_select(W.WEDLM_BF16, B, Wn, V, z, filled, lam, tau, min_fill, o["entropy"],
                           o["score"], o["argmax"], o["selected"], ws, nbytes)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in o.items()}


def _noalloc_form(B, Wn, V, z, filled, lam, tau, min_fill):
    o = _outputs(B, Wn)
    W.wedlm_entropy_select_noalloc(W.WEDLM_BF16, B, Wn, V, z, filled, lam, tau, min_fill,
                                   o["entropy"], o["score"], o["argmax"], o["selected"])
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in o.items()}


def test_noalloc_matches_workspace_form():
    lam, tau, min_fill = 0.1, 1.0, 1
    cases = [
        # (B, W, V, seed, spike, aligned): the streaming workload's shape first
        (16, 16, 151936, 1, (6.0, 12.0), True),
        (3, 8, 5000, 2, (16.0, 20.0), True),     # smaller: stale partials stay behind it
        (2, 5, 3001, 3, (0.0, 12.0), False),     # rows 16-byte misaligned: element path
    ]
    for B, Wn, V, seed, spike, aligned in cases:
        print(f"[noalloc] B={B} W={Wn} V={V} aligned={aligned}", flush=True)
        z, filled = _inputs(B, Wn, V, seed, spike)
        if not aligned:
            # the same values one element into a larger buffer
            buf = torch.empty(B * Wn * V + 1, dtype=torch.bfloat16, device="cuda")
            buf[1:].copy_(z.reshape(-1))
            z = buf[1:].view(B, Wn, V)
            assert z.data_ptr() % 16 != 0
        ref = _workspace_form(B, Wn, V, z, filled, lam, tau, min_fill)
        got = _noalloc_form(B, Wn, V, z, filled, lam, tau, min_fill)
        for key in ref:
            assert np.array_equal(got[key], ref[key]), (key, B, Wn, V)
        assert np.isfinite(got["entropy"]).all()
        if B * Wn * V <= 200000:
            # the oracle's bar on the smaller calls
            H, a = oracle.vocab_entropy_argmax(z.float().cpu().numpy())
            assert (np.abs(got["entropy"] - H) <= 1e-3).all()
            assert np.array_equal(got["argmax"], a)
            f = filled.cpu().numpy().astype(bool)
            for b in range(B):
                r = oracle.select_slots(H[b], f[b], lam, tau, min_fill,
                                        adopt=got["selected"][b].astype(bool))
                assert np.array_equal(got["selected"][b].astype(bool), r["selected"]), b
    print("[noalloc] workspace-free calls bitwise equal to the workspace form", flush=True)


def test_noalloc_refuses_sizes_beyond_its_scratch():
    # 1000 x 64 rows of a 152k vocabulary need ~10 MB of partials: refused
    # before anything is enqueued, with its own status
    z = torch.empty(16, dtype=torch.bfloat16, device="cuda")
    filled = torch.zeros(16, dtype=torch.uint8, device="cuda")
    o = _outputs(1, 16)
    with pytest.raises(W.WedlmError) as e:
        W.wedlm_entropy_select_noalloc(W.WEDLM_BF16, 1000, 64, 151936, z, filled, 0.1, 1.0, 1,
                                       o["entropy"], o["score"], o["argmax"], o["selected"])
    assert e.value.status == -5
