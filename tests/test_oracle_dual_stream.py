"""Pins for the oracle's dual-stream masking attention (CPU).

The explicit-mask form is checked against a second, independent form built
from the window-step oracle: each block of the prediction stream is
topologically reordered and attended causally over [memory prefix of the
preceding blocks ; the block], and the memory stream is the same with every
position observed. Also: no leakage (a prediction token's output does not
move when memory tokens of its own or later blocks, or prediction tokens of
other blocks, change), one all-observed block equals plain causal attention
(torch's scaled_dot_product_attention in float64), and the rank inside a
block is the stable partition.
"""

import numpy as np
import torch

from oracle import rope_rotate, topological_reorder, window_attention_reordered
from oracle.dual_stream import block_rank, dual_stream_attention, dual_stream_visibility


def _inputs(seed, N=48, Hq=4, Hkv=2, D=16):
    rng = np.random.default_rng(seed)
    x = lambda h: rng.standard_normal((N, h, D))
    return (x(Hq), x(Hkv), x(Hkv), x(Hq), x(Hkv), x(Hkv), rng.random(N) < 0.5)


def _reordered_form(qm, km, vm, qp, kp, vp, filled, block, theta):
    N = qm.shape[0]
    pos = np.arange(N)[:, None]
    kmr = rope_rotate(km, pos, theta)
    out_m = np.empty_like(qm)
    out_p = np.empty_like(qp)
    for j0 in range(0, N, block):
        j1 = min(j0 + block, N)
        for f_blk, (q, k, v), out in (
                (np.ones(j1 - j0, bool), (qm, km, vm), out_m),
                (filled[j0:j1], (qp, kp, vp), out_p)):
            r = topological_reorder(f_blk, j0)
            perm, ppos = np.asarray(r["perm"]), np.asarray(r["pos"])
            o = window_attention_reordered(rope_rotate(q[j0:j1][perm], ppos[:, None], theta),
                                           rope_rotate(k[j0:j1][perm], ppos[:, None], theta),
                                           v[j0:j1][perm], kmr[:j0], vm[:j0])
            out[j0 + perm] = o
    return out_m, out_p


def test_mask_form_equals_reordered_form():
    for seed, block in ((0, 8), (1, 16), (2, 48), (3, 5)):
        args = _inputs(seed)
        om, op = dual_stream_attention(*args, block, theta=1e4)
        rm, rp = _reordered_form(*args, block, 1e4)
        assert np.abs(om - rm).max() < 1e-12 and np.abs(op - rp).max() < 1e-12, (seed, block)


def test_no_leakage():
    qm, km, vm, qp, kp, vp, f = _inputs(4)
    block = 8
    _, base = dual_stream_attention(qm, km, vm, qp, kp, vp, f, block, 1e4)
    rng = np.random.default_rng(5)
    for j0 in (0, 8, 24, 40):
        km2, vm2, kp2, vp2 = km.copy(), vm.copy(), kp.copy(), vp.copy()
        km2[j0:] += rng.standard_normal(km2[j0:].shape)   # memory of this and later blocks
        vm2[j0:] += rng.standard_normal(vm2[j0:].shape)
        other = np.ones(48, bool)
        other[j0:j0 + block] = False
        kp2[other] += rng.standard_normal(kp2[other].shape)  # prediction tokens of other blocks
        vp2[other] += rng.standard_normal(vp2[other].shape)
        _, moved = dual_stream_attention(qm, km2, vm2, qp, kp2, vp2, f, block, 1e4)
        assert np.array_equal(moved[j0:j0 + block], base[j0:j0 + block]), j0


def test_one_observed_block_is_causal_attention():
    qm, km, vm, _, _, _, _ = _inputs(6, N=20, Hq=2, Hkv=2)
    om, op = dual_stream_attention(qm, km, vm, qm, km, vm, np.ones(20, bool), 20, 1e4)
    pos = np.arange(20)[:, None]
    q = torch.from_numpy(rope_rotate(qm, pos, 1e4)).permute(1, 0, 2)
    k = torch.from_numpy(rope_rotate(km, pos, 1e4)).permute(1, 0, 2)
    v = torch.from_numpy(vm).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
    ref = ref.permute(1, 0, 2).numpy()
    assert np.abs(om - ref).max() < 1e-12 and np.abs(op - ref).max() < 1e-12


def test_block_rank_and_visibility_counts():
    f = np.array([0, 1, 1, 0, 1, 0, 0, 1], bool)
    assert block_rank(f, 4).tolist() == [2, 0, 1, 3, 0, 2, 3, 1]
    vis = dual_stream_visibility(f, 4)
    # memory row t sees t + 1 keys; prediction row t sees its block start plus its rank + 1
    assert vis[:8].sum(axis=1).tolist() == list(range(1, 9))
    assert vis[8:].sum(axis=1).tolist() == [3, 1, 2, 4, 5, 7, 8, 6]
