"""The fused step tail (wedlm_select_commit_reorder) against the three calls it
replaces, through the C ABI.

On the same state and logits, wedlm_entropy_select, the window-state half of
wedlm_commit_prefix_rope (k = v = NULL) and wedlm_window_reorder_rule must
give bitwise the same outputs as the one fused call: both run the same
per-sequence device functions, so nothing - not even a float's last bit - may
differ. Cases cover W from 1 to 64, the commit clamp at the end of the page
table, negative prefix lengths, empty and full windows, both commit rules,
min_fill 0 / 1, thresholds of +-inf, f32 and bf16 logits, and a logits tensor
that is not 16-byte aligned (scalar path); three tails are chained per case.
The fused tail's end-to-end parity with the oracle is in test_gpu_stream.py.
"""

import zlib

import numpy as np
import pytest
import torch

from causal_streaming_decoding_amd import wedlm as W_

pytestmark = pytest.mark.gpu

P = 16
MASK = -1

# name, B, W, V, max_pages, dtype, lam, tau, min_fill, rule, offset
CASES = [
    ("w16_stream", 8, 16, 3001, 6, torch.bfloat16, 0.1, 1.5, 1, W_.COMMIT_STREAM, 0),
    ("w64_clamp", 5, 64, 1024, 5, torch.bfloat16, 0.05, 2.5, 1, W_.COMMIT_STREAM, 0),
    ("w1", 7, 1, 777, 3, torch.float32, 0.0, 0.5, 1, W_.COMMIT_STREAM, 0),
    ("w33_block", 6, 33, 2048, 6, torch.bfloat16, 0.02, 3.0, 1, W_.COMMIT_BLOCK, 0),
    ("w7_nofloor", 9, 7, 4099, 2, torch.float32, 0.2, 0.3, 0, W_.COMMIT_STREAM, 0),
    ("w16_one_by_one", 4, 16, 512, 4, torch.bfloat16, 0.1, float("-inf"), 1, W_.COMMIT_STREAM, 0),
    ("w16_all", 4, 16, 512, 4, torch.bfloat16, 0.1, float("inf"), 1, W_.COMMIT_BLOCK, 0),
    ("w12_unaligned", 3, 12, 1000, 3, torch.bfloat16, 0.1, 2.0, 1, W_.COMMIT_STREAM, 1),
]


def _state(B, W, max_pages, gen):
    dev = "cuda"
    filled = (torch.rand((B, W), generator=gen) < 0.45).to(torch.uint8)
    filled[0] = 1                   # a full window
    if B > 1:
        filled[1] = 0               # an empty one
    if B > 2:
        filled[2, : max(W // 2, 1)] = 1  # a long leading run
    tokens = torch.randint(0, 50000, (B, W), generator=gen, dtype=torch.int32)
    tokens = torch.where(filled.bool(), tokens, torch.full_like(tokens, MASK))
    cap = max_pages * P
    prefix = torch.randint(0, cap + 1, (B,), generator=gen, dtype=torch.int32)
    prefix[0] = cap - 3             # the commit is clamped to the pages left
    if B > 3:
        prefix[3] = -5              # read as 0
    if B > 4:
        prefix[4] = cap             # table full: nothing can be committed
    num_pages = B * max_pages
    table = torch.randperm(num_pages, generator=gen).to(torch.int32).view(B, max_pages)
    return {"tokens": tokens.to(dev), "filled": filled.to(dev), "prefix_len": prefix.to(dev),
            "table": table.to(dev), "num_pages": num_pages}


def _logits(B, W, V, dtype, offset, gen):
    z = torch.randn((B, W, V), generator=gen) * 2.0
    # low-entropy slots: a spike on one token so that some scores clear tau
    spike = torch.rand((B, W), generator=gen) < 0.4
    tok = torch.randint(0, V, (B, W), generator=gen)
    z[spike, tok[spike]] += 18.0
    flat = torch.empty(B * W * V + offset, dtype=dtype, device="cuda")
    flat[offset:] = z.reshape(-1).to(dtype).cuda()
    return flat[offset:].view(B, W, V)


def _outputs(B, W):
    i32 = dict(dtype=torch.int32, device="cuda")
    return {"entropy": torch.full((B, W), float("nan"), device="cuda"),
            "score": torch.full((B, W), float("nan"), device="cuda"),
            "argmax": torch.full((B, W), -7, **i32),
            "selected": torch.full((B, W), 7, dtype=torch.uint8, device="cuda"),
            "commit_len": torch.full((B,), -7, **i32),
            "cache_slot": torch.full((B, W), -7, **i32),
            "perm": torch.full((B, W), -7, **i32), "inv": torch.full((B, W), -7, **i32),
            "pos": torch.full((B, W), -7, **i32), "n_obs": torch.full((B,), -7, **i32),
            "run_len": torch.full((B,), -7, **i32)}


def _reorder(B, W, rule, st, o):
    W_.wedlm_window_reorder_rule(B, W, rule, st["filled"], st["prefix_len"], o["perm"], o["inv"],
                                 o["pos"], o["n_obs"], o["run_len"])


def _separate(case, st, o, logits, ws, caches):
    name, B, W, V, max_pages, dtype, lam, tau, min_fill, rule, _ = case
    dt = W_.dtype_code(dtype)
    W_.wedlm_entropy_select(dt, B, W, V, logits, st["filled"], lam, tau, min_fill, o["entropy"],
                            o["score"], o["argmax"], o["selected"], ws, ws.numel())
    W_.wedlm_commit_prefix_rope(dt, 1, B, W, 1, 128, P, st["num_pages"], max_pages, 1e4,
                                o["run_len"], o["selected"], o["argmax"], None, None, st["table"],
                                caches[0], caches[1], st["tokens"], st["filled"],
                                st["prefix_len"], o["commit_len"], o["cache_slot"], MASK)
    _reorder(B, W, rule, st, o)


def _fused(case, st, o, logits, ws):
    name, B, W, V, max_pages, dtype, lam, tau, min_fill, rule, _ = case
    W_.wedlm_select_commit_reorder(W_.dtype_code(dtype), B, W, V, logits, lam, tau, min_fill, P,
                                   st["num_pages"], max_pages, rule, st["table"], o["run_len"],
                                   st["tokens"], st["filled"], st["prefix_len"], o["commit_len"],
                                   o["cache_slot"], MASK, o["entropy"], o["score"], o["argmax"],
                                   o["selected"], o["perm"], o["inv"], o["pos"], o["n_obs"], ws,
                                   ws.numel())


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fused_tail_bitwise_equals_separate_calls(case):
    name, B, W, V, max_pages, dtype, lam, tau, min_fill, rule, offset = case
    print(f"[tail] {name} B={B} W={W} V={V} rule={rule}", flush=True)
    gen = torch.Generator().manual_seed(zlib.crc32(name.encode()))
    a = _state(B, W, max_pages, gen)
    b = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in a.items()}
    oa, ob = _outputs(B, W), _outputs(B, W)
    caches = (torch.zeros(16, dtype=dtype, device="cuda"),
              torch.zeros(16, dtype=dtype, device="cuda"))
    ws_bytes = W_.wedlm_entropy_select_workspace_size(W_.dtype_code(dtype), B, W, V)
    wsa = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    wsb = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    # both sides start from the same order
    _reorder(B, W, rule, a, oa)
    _reorder(B, W, rule, b, ob)
    committed = 0
    for it in range(3):
        logits = _logits(B, W, V, dtype, offset, gen)
        _separate(case, a, oa, logits, wsa, caches)
        _fused(case, b, ob, logits, wsb)
        torch.cuda.synchronize()
        for key in ("tokens", "filled", "prefix_len"):
            assert torch.equal(a[key], b[key]), (name, it, key)
        for key in oa:
            assert torch.equal(_bits(oa[key]), _bits(ob[key])), (name, it, key)
        committed += int(oa["commit_len"].sum())
        sel = oa["selected"].cpu().numpy()
        assert set(np.unique(sel)) <= {0, 1}
    # clamp: the sequence three positions before the end of its table commits at most 3
    cap = max_pages * P
    assert int(a["prefix_len"][0]) <= cap
    assert (a["prefix_len"].cpu().numpy() <= cap).all()
    print(f"[tail] {name}: 3 tails bitwise equal, committed {committed}", flush=True)


def test_fused_tail_rejects_small_workspace():
    B, W, V = 2, 8, 100
    ws_bytes = W_.wedlm_entropy_select_workspace_size(W_.WEDLM_BF16, B, W, V)
    st = _state(B, W, 2, torch.Generator().manual_seed(3))
    o = _outputs(B, W)
    logits = torch.zeros((B, W, V), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(ws_bytes - 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(W_.WedlmError) as e:
        W_.wedlm_select_commit_reorder(W_.WEDLM_BF16, B, W, V, logits, 0.1, 1.0, 1, P,
                                       st["num_pages"], 2, W_.COMMIT_STREAM, st["table"],
                                       o["run_len"], st["tokens"], st["filled"],
                                       st["prefix_len"], o["commit_len"], o["cache_slot"], MASK,
                                       o["entropy"], o["score"], o["argmax"], o["selected"],
                                       o["perm"], o["inv"], o["pos"], o["n_obs"], ws, ws.numel())
    assert e.value.status == -3
