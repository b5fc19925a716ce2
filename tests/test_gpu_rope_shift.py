"""RoPE shift invariance on the device: every logical position moved by c (GPU).

Rotary embedding makes the score of a query and a key depend only on the
difference of their positions (RoFormer, listed under "Builds on" on the
mlsanity.com page on WeDLM; the sai.science review's "Summary": the decoder
keeps logical positions through RoPE). So when every position of a window step
- the cached prefix keys and the window's rows - moves by the same c, the
attention output is unchanged.

Per shift c the raw prefix keys are rotated on the GPU at t + c
(``wedlm_rope_logical`` with the identity order, 64 positions per call row)
and written into the paged cache, then the window attends with the reorder's
positions + c, once through the fused call (``wedlm_window_attn_rope``: its own
device RoPE on the window rows) and once through the separate pass
(``wedlm_rope_logical`` + ``wedlm_window_attn``). Checks:

* every rotated row the GPU stores at the shifted positions - the prefix keys
  from the separate pass, the window's q/k from the separate pass, and the
  committed window keys the fused call appends to the cache - against the
  float64 rotation at those positions, within one rounding to the storage type;
* both attention outputs against the float64 oracle of the shifted problem
  (the oracle rotates the same raw rows itself and stores them through the
  storage type): the attention bar;
* fp32 storage: each output against the unshifted one within 1e-4 (+1e-4
  relative), so a rotation angle off by ~1e-4 rad anywhere fails. (With bf16
  storage the rows are rounded at different angles, which moves the output
  by up to ~7e-3 in the float64 oracle itself: there the comparisons with the
  oracle above carry the check.)

The shifts reach 2^24 + 17, where an angle formed in fp32 would be off by
about one radian.
"""

import dataclasses

import numpy as np
import pytest
import torch

from causal_streaming_decoding_amd import layout
from causal_streaming_decoding_amd import wedlm as Wd
from oracle.attention import window_attention_masked
from oracle.rope import rope_rotate

from .parity import ATTN_ATOL, ATTN_RTOL, storage_rounding, stored_rotation_bound

pytestmark = pytest.mark.gpu

SHIFTS = (1, 4093, 1_000_003, (1 << 24) + 17)
PAGE = 16
CHUNK = 64


@dataclasses.dataclass(frozen=True)
class Case:
    name: str
    dtype: str
    Hq: int
    Hkv: int
    D: int
    W: int
    theta: float
    prefix: tuple


CASES = [
    # key-range splits (few groups), an empty prefix, a ragged last page
    Case("bf16_g4_W16", "bf16", 8, 2, 128, 16, 1e6, (0, 37, 700)),
    # 224 query rows per group: four row parts
    Case("bf16_g7_W32", "bf16", 14, 2, 128, 32, 1e6, (129, 1000)),
    Case("f32_g2_W8", "f32", 4, 2, 64, 8, 1e4, (5, 40)),
]


def _torch_dtype(dt):
    return torch.bfloat16 if dt == "bf16" else torch.float32


def _inputs(case, seed):
    """Raw (unrotated) prefix keys and values, window rows and flags, in the storage type."""
    rng = np.random.default_rng(seed)
    td = _torch_dtype(case.dtype)
    B = len(case.prefix)

    def stored(x):
        return torch.from_numpy(x).to(td)

    pre_k = [stored(rng.standard_normal((L, case.Hkv, case.D))) for L in case.prefix]
    pre_v = [stored(rng.standard_normal((L, case.Hkv, case.D))) for L in case.prefix]
    q = stored(rng.standard_normal((1, B, case.W, case.Hq, case.D)))
    k = stored(rng.standard_normal((1, B, case.W, case.Hkv, case.D)))
    v = stored(rng.standard_normal((1, B, case.W, case.Hkv, case.D)))
    filled = rng.random((B, case.W)) < 0.5
    filled[0, 0] = True
    filled[-1, :3] = True  # a committed run of at least 3
    # every sequence's pages (prefix + window), shuffled over one pool
    n_pages = [(L + case.W + PAGE - 1) // PAGE for L in case.prefix]
    max_pages = max(1, max(n_pages))
    pool = rng.permutation(sum(n_pages) + 1)
    bt = np.zeros((B, max_pages), np.int32)
    at = 0
    for b, n in enumerate(n_pages):
        bt[b, :n] = pool[at:at + n]
        at += n
    return dict(pre_k=pre_k, pre_v=pre_v, q=q, k=k, v=v, filled=filled, block_table=bt,
                num_pages=len(pool))


def _rotate_prefix_on_gpu(case, pre_k, c, dev):
    """Rotated prefix keys per sequence, [L, Hkv, D], by wedlm_rope_logical at t + c."""
    td = _torch_dtype(case.dtype)
    rows = []  # (sequence, start)
    for b, L in enumerate(case.prefix):
        rows += [(b, s) for s in range(0, L, CHUNK)]
    if not rows:
        return [torch.empty((0, case.Hkv, case.D), dtype=td, device=dev) for _ in case.prefix]
    n = len(rows)
    kin = torch.zeros((1, n, CHUNK, case.Hkv, case.D), dtype=td)
    pos = np.zeros((n, CHUNK), np.int32)
    for r, (b, s) in enumerate(rows):
        m = min(CHUNK, case.prefix[b] - s)
        kin[0, r, :m] = pre_k[b][s:s + m]
        pos[r] = s + c + np.arange(CHUNK)
    kin = kin.to(dev)
    perm = torch.arange(CHUNK, dtype=torch.int32, device=dev).repeat(n, 1).contiguous()
    pos_d = torch.from_numpy(pos).to(dev)
    qo = torch.empty_like(kin)
    ko = torch.empty_like(kin)
    vo = torch.empty_like(kin)
    # the keys ride as the query rows too (Hq = Hkv); only k_phys is used
    Wd.wedlm_rope_logical(Wd.dtype_code(td), 1, n, CHUNK, case.Hkv, case.Hkv, case.D,
                          case.theta, kin, kin, kin, perm, pos_d, qo, ko, vo)
    out = []
    for b, L in enumerate(case.prefix):
        parts = [ko[0, r, :min(CHUNK, L - s)] for r, (bb, s) in enumerate(rows) if bb == b]
        out.append(torch.cat(parts) if parts else
                   torch.empty((0, case.Hkv, case.D), dtype=td, device=dev))
    return out


def _gpu_outputs(case, inp, c, dev):
    """Everything the GPU computes with every position shifted by c (host copies):
    attention outputs in physical order (fused, separate), the reorder's perm and
    run, the rotated prefix keys, the separate pass's q/k rows, and the rows the
    fused call appends at positions L .. L + run - 1."""
    td = _torch_dtype(case.dtype)
    code = Wd.dtype_code(td)
    B, W = len(case.prefix), case.W
    bt = torch.from_numpy(inp["block_table"]).to(dev)
    max_pages = bt.shape[1]
    kc, vc = layout.alloc_caches(1, inp["num_pages"], case.Hkv, case.D, PAGE, td, dev)
    rot = _rotate_prefix_on_gpu(case, inp["pre_k"], c, dev)
    for b, L in enumerate(case.prefix):
        layout.write_rows(kc, vc, 0, bt[b], 0, rot[b], inp["pre_v"][b].to(dev))

    filled = torch.from_numpy(inp["filled"].astype(np.uint8)).to(dev)
    prefix_len = torch.tensor(case.prefix, dtype=torch.int32, device=dev)
    perm = torch.empty((B, W), dtype=torch.int32, device=dev)
    inv = torch.empty_like(perm)
    pos = torch.empty_like(perm)
    n_obs = torch.empty(B, dtype=torch.int32, device=dev)
    run = torch.empty_like(n_obs)
    Wd.wedlm_window_reorder(B, W, filled, prefix_len, perm, inv, pos, n_obs, run)
    pos_c = (pos.to(torch.int64) + c).to(torch.int32).contiguous()

    q, k, v = (x.to(dev).contiguous() for x in (inp["q"], inp["k"], inp["v"]))
    max_prefix = max(case.prefix)
    ws_bytes = Wd.wedlm_window_attn_workspace_size(code, 1, B, W, case.Hq, case.Hkv, case.D,
                                                   PAGE, max_prefix)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    scale = 1.0 / np.sqrt(case.D)

    fused = torch.empty((1, B, W, case.Hq, case.D), dtype=td, device=dev)
    Wd.wedlm_window_attn_rope(code, 1, B, W, case.Hq, case.Hkv, case.D, PAGE, inp["num_pages"],
                              max_pages, max_prefix, scale, case.theta, q, k, v, perm, pos_c,
                              kc, vc, bt, prefix_len, run, fused, ws, ws_bytes)

    qp = torch.empty_like(q)
    kp = torch.empty_like(k)
    vp = torch.empty_like(v)
    Wd.wedlm_rope_logical(code, 1, B, W, case.Hq, case.Hkv, case.D, case.theta, q, k, v, perm,
                          pos_c, qp, kp, vp)
    sep = torch.empty_like(fused)
    Wd.wedlm_window_attn(code, 1, B, W, case.Hq, case.Hkv, case.D, PAGE, inp["num_pages"],
                         max_pages, max_prefix, scale, qp, kp, vp, kc, vc, bt, prefix_len, sep,
                         ws, ws_bytes)
    torch.cuda.synchronize()
    run_h = run.cpu().numpy()
    appended = []
    for b, L in enumerate(case.prefix):
        kr, vr = layout.read_rows(kc, vc, 0, bt[b], L, int(run_h[b]))
        appended.append((kr.double().cpu().numpy(), vr.double().cpu().numpy()))
    host = lambda t: t.double().cpu().numpy()
    return dict(fused=host(fused[0]), separate=host(sep[0]), perm=perm.cpu().numpy(),
                run=run_h, prefix_k=[host(r) for r in rot], q_phys=host(qp[0]),
                k_phys=host(kp[0]), appended=appended)


def _oracle(case, inp, c, perm):
    """float64 rotations at the shifted positions and the attention of the shifted
    problem (physical order)."""
    keep = storage_rounding(case.dtype) or (lambda x: x)
    B = len(case.prefix)
    out = np.empty((B, case.W, case.Hq, case.D))
    ref = dict(prefix_k=[], q_slot=[], k_slot=[])
    for b, L in enumerate(case.prefix):
        pk = inp["pre_k"][b].double().numpy()
        pv = inp["pre_v"][b].double().numpy()
        k_cache = rope_rotate(pk, (np.arange(L) + c)[:, None], case.theta)
        slot_pos = (L + c + np.arange(case.W))[:, None]
        q = rope_rotate(inp["q"][0, b].double().numpy(), slot_pos, case.theta)
        k = rope_rotate(inp["k"][0, b].double().numpy(), slot_pos, case.theta)
        v = inp["v"][0, b].double().numpy()
        ref["prefix_k"].append(k_cache)
        ref["q_slot"].append(q)
        ref["k_slot"].append(k)
        o = window_attention_masked(keep(q), keep(k), v, inp["filled"][b], keep(k_cache), pv)
        out[b] = o[perm[b]]
    ref["attn"] = out
    return ref


def _check_rows(got, ref, dtype, what):
    err = np.abs(got - ref)
    assert np.all(err <= stored_rotation_bound(ref, dtype)), (what, float(err.max()))


@pytest.mark.parametrize("case", CASES, ids=lambda c: c.name)
def test_attention_is_invariant_under_a_position_shift(case):
    print(f"[rope-shift] {case.name}", flush=True)
    dev = "cuda"
    inp = _inputs(case, seed=7)
    base = _gpu_outputs(case, inp, 0, dev)
    perm = base["perm"]
    for c in (0,) + SHIFTS:
        got = _gpu_outputs(case, inp, c, dev) if c else base
        assert np.array_equal(got["perm"], perm)
        ref = _oracle(case, inp, c, perm)
        for b, L in enumerate(case.prefix):
            _check_rows(got["prefix_k"][b], ref["prefix_k"][b], case.dtype, (c, b, "prefix k"))
            _check_rows(got["q_phys"][b], ref["q_slot"][b][perm[b]], case.dtype, (c, b, "q"))
            _check_rows(got["k_phys"][b], ref["k_slot"][b][perm[b]], case.dtype, (c, b, "k"))
            n = int(got["run"][b])
            kr, vr = got["appended"][b]
            _check_rows(kr, ref["k_slot"][b][:n], case.dtype, (c, b, "appended k"))
            assert np.array_equal(vr, inp["v"][0, b, :n].double().numpy()), (c, b)
        bar = ATTN_ATOL + ATTN_RTOL * np.abs(ref["attn"])
        for name in ("fused", "separate"):
            err = np.abs(got[name] - ref["attn"])
            assert np.all(err <= bar), (case.name, c, name, float(err.max()))
            msg = f"max |out - oracle| {err.max():.2e}"
            if c:
                d = np.abs(got[name] - base[name])
                if case.dtype == "f32":
                    assert np.all(d <= 1e-4 + 1e-4 * np.abs(base[name])), (c, name, float(d.max()))
                msg += f", max |out(c) - out(0)| {d.max():.2e}"
            print(f"[rope-shift] {case.name} c={c} {name}: {msg}", flush=True)
    print(f"[rope-shift] {case.name}: committed runs {got['run'].tolist()}", flush=True)
