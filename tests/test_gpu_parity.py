"""GPU window step against the fp64 oracle, through the C ABI (needs an MI355X).

Each workload's inputs are drawn by the seeded generator on the host, uploaded,
run through the five entry points, and compared output by output with the
oracle on identical values (bars in tests/parity.py).
"""

import dataclasses

import numpy as np
import pytest
import torch

from causal_streaming_decoding_amd import workloads as WL
from causal_streaming_decoding_amd.synth import make_step_inputs

from .parity import compare_step, gpu_step, oracle_step, stored_pair_bound

pytestmark = pytest.mark.gpu


def _check(wl, seed=None, layers=None, steps=1):
    """Both forms of the step - separate RoPE pass and RoPE fused into attention
    and commit - against one oracle run, and against each other."""
    print(f"[parity] {wl.name} seed={seed}", flush=True)
    inp = make_step_inputs(wl, seed=seed, steps=steps)
    gpu = gpu_step(wl, inp)
    fused = gpu_step(wl, inp, fused_rope=True)
    ref = oracle_step(wl, inp, gpu=gpu, layers=layers)
    rep = compare_step(wl, gpu, ref, layers=layers)
    rep_f = compare_step(wl, fused, ref, layers=layers)
    # the selection and state never depend on the RoPE form
    for key in ("perm", "run", "entropy", "argmax", "selected", "commit_len", "cache_slot",
                "tokens", "filled", "prefix_len"):
        assert np.array_equal(gpu[key], fused[key]), key
    print(f"[parity] {wl.name}: {rep}; fused {rep_f}", flush=True)
    return rep


def test_tiny_fp32():
    _check(WL.TINY_FP32)


def test_tiny_fp32_other_seeds():
    for seed in (1, 2, 3):
        _check(WL.TINY_FP32, seed=seed)


def test_qwen3_8b_bs1_L2048():
    _check(WL.QWEN3_8B_BS1)


def test_qwen25_7b_bs16_ragged():
    _check(WL.QWEN25_7B_RAGGED)


def test_qwen3_8b_bs4_L32768():
    _check(WL.QWEN3_8B_LONG)


def _variant(base, **kw):
    return dataclasses.replace(base, **kw)


@pytest.mark.parametrize("name,wl", [
    ("empty_prefix", _variant(WL.QWEN3_8B_BS1, name="edge_empty_prefix", prefix=("fixed", 0),
                              V=4096, B=2)),
    ("ragged_tail", _variant(WL.QWEN3_8B_BS1, name="edge_ragged_tail", prefix=("fixed", 77),
                             V=4100, B=3)),
    ("w64_max_rows", _variant(WL.QWEN3_8B_BS1, name="edge_w64", W=64, Hq=16, Hkv=4,
                              prefix=("fixed", 300), V=2048, B=2)),
    ("w1", _variant(WL.QWEN3_8B_BS1, name="edge_w1", W=1, prefix=("fixed", 33), V=1000, B=2,
                    fill=("count", 1))),
    ("all_filled", _variant(WL.QWEN3_8B_BS1, name="edge_all_filled", fill=("count", 16),
                            prefix=("fixed", 129), V=3000, B=2)),
    ("no_filled", _variant(WL.QWEN3_8B_BS1, name="edge_no_filled", fill=("none",),
                           prefix=("fixed", 1000), V=3000, B=2)),
    ("mha", _variant(WL.QWEN3_8B_BS1, name="edge_mha", Hq=8, Hkv=8, prefix=("fixed", 513),
                     V=2000, B=2)),
    ("gqa7_split_ragged", _variant(WL.QWEN25_7B_RAGGED, name="edge_gqa7_small", B=3,
                                   prefix=("uniform", 1, 700), V=5000)),
    ("low_entropy_threshold_fires", _variant(WL.QWEN3_8B_BS1, name="edge_low_entropy",
                                             spike=("all_uniform", 16.0, 20.0), V=4096, B=4)),
    ("tiny_fp32_multi_layer", _variant(WL.TINY_FP32, name="edge_fp32_layers", n_layers=3, B=3,
                                       prefix=("uniform", 0, 45))),
    ("stream_shape_short", _variant(WL.QWEN3_8B_STREAM, name="edge_stream_layers", n_layers=3,
                                    B=4, V=3000, fill=("frac", 0.0, 1.0), steps=1)),
    # 128 query rows: two 4-wave row parts per work unit, split key range
    ("nw8_split", _variant(WL.QWEN3_8B_BS1, name="edge_nw8_split", W=32, prefix=("fixed", 3000),
                           V=2048, B=2, fill=("frac", 0.3, 0.7))),
    # 128 query rows in two row parts, no split (512 groups), short ragged prefixes
    ("nw8_many_groups", _variant(WL.QWEN3_8B_STREAM, name="edge_nw8_layers", n_layers=8, B=8, W=32,
                                 V=2048, fill=("frac", 0.0, 1.0), prefix=("uniform", 17, 900),
                                 steps=1)),
    # 224 rows: four 4-wave row parts per work unit, short splits
    ("rowparts_short_splits", _variant(WL.QWEN25_7B_RAGGED, name="edge_rowparts_short", B=2,
                                   prefix=("uniform", 40, 130), V=2048)),
    # split plan over very uneven prefixes: empty, one key, one page, a long one
    ("split_plan_extremes", _variant(WL.QWEN25_7B_RAGGED, name="edge_split_extremes", B=6,
                                     prefix=("list", (0, 1, 4000, 16, 2047, 33)), V=2048)),
    # two row parts, split plan with a sequence that has no prefix at all
    ("split_plan_nw8", _variant(WL.QWEN3_8B_BS1, name="edge_split_nw8", W=32, B=3,
                                prefix=("list", (3000, 5, 0)), V=2048, fill=("frac", 0.3, 0.7))),
    # 4-wave workgroups, 40 sequences sharing 160 workgroups per kv head
    ("split_plan_many_seqs", _variant(WL.QWEN3_8B_BS1, name="edge_split_many", B=40,
                                      prefix=("uniform", 0, 1500), V=1024)),
    # more sequences than one wavefront's lanes: the plan scans them in chunks
    ("split_plan_100_seqs", _variant(WL.QWEN3_8B_BS1, name="edge_split_100", B=100,
                                     prefix=("uniform", 0, 300), V=512)),
])
def test_edge_cases(name, wl):
    _check(wl)


@pytest.mark.parametrize("wl", [
    # one sequence per page count: splits, a ragged last page, 4 row tiles
    _variant(WL.QWEN3_8B_BS1, name="poison_bs1", B=3, prefix=("list", (77, 2047, 1000)), V=2048),
    # 224 rows (one wide workgroup per split), ragged prefixes over split key ranges
    _variant(WL.QWEN25_7B_RAGGED, name="poison_gqa7", B=4, prefix=("uniform", 1, 900), V=2048),
    # no split (many groups)
    _variant(WL.QWEN3_8B_STREAM, name="poison_layers", n_layers=6, B=6, V=2048,
             fill=("frac", 0.0, 1.0), prefix=("uniform", 17, 500), steps=1),
    _variant(WL.TINY_FP32, name="poison_fp32", B=3, prefix=("list", (40, 3, 17))),
], ids=lambda w: w.name)
def test_non_finite_page_tails_never_reach_the_output(wl):
    # cache positions a sequence has not written (past prefix_len in its last
    # page) hold NaN / Inf: both step forms still match the oracle
    print(f"[parity] {wl.name}: NaN / Inf page tails", flush=True)
    inp = make_step_inputs(wl)
    gpu = gpu_step(wl, inp, poison=True)
    fused = gpu_step(wl, inp, fused_rope=True, poison=True)
    ref = oracle_step(wl, inp, gpu=gpu)
    for out in (gpu, fused):
        assert np.isfinite(out["attn_out_phys"]).all()
        compare_step(wl, out, ref)


def test_deterministic_bitwise():
    wl = _variant(WL.QWEN25_7B_RAGGED, name="determinism", B=4, V=20000)
    inp = make_step_inputs(wl)
    for fused in (False, True):
        a = gpu_step(wl, inp, fused_rope=fused)
        b = gpu_step(wl, inp, repeat=2, fused_rope=fused)
        keys = ["attn_out_phys", "entropy", "score", "tokens", "cache_slot"]
        if not fused:
            keys.append("q_phys")
        for key in keys:
            assert np.array_equal(a[key], b[key]), (key, fused)
        for rk in a["committed_rows"]:
            assert np.array_equal(a["committed_rows"][rk][0], b["committed_rows"][rk][0]), rk


@pytest.mark.parametrize("wl", [
    _variant(WL.QWEN3_8B_BS1, name="append_forms_bf16", fill=("count", 9), prefix=("fixed", 45),
             V=2048, B=3),
    _variant(WL.QWEN3_8B_BS1, name="append_forms_w64", W=64, Hq=16, Hkv=4, fill=("count", 64),
             prefix=("fixed", 77), V=2048, B=2),  # all filled: 64 rows over 4 chunks, 256-row groups
    _variant(WL.TINY_FP32, name="append_forms_fp32", n_layers=2, B=3, fill=("count", 5)),
])
def test_fused_commit_forms_agree(wl):
    """The committed rows appended by the fused attention call and those the
    fused commit call writes itself: same state, rows within one storage ulp."""
    print(f"[parity] {wl.name}", flush=True)
    inp = make_step_inputs(wl)
    a = gpu_step(wl, inp, fused_rope=True, append=True)
    b = gpu_step(wl, inp, fused_rope=True, append=False)
    for key in ("commit_len", "cache_slot", "tokens", "filled", "prefix_len", "attn_out_phys"):
        assert np.array_equal(a[key], b[key]), key
    assert a["committed_rows"].keys() == b["committed_rows"].keys()
    assert int(a["commit_len"].max()) > 0
    for rk, (ka, va) in a["committed_rows"].items():
        kb, vb = b["committed_rows"][rk]
        assert np.array_equal(va, vb), rk
        assert (np.abs(ka - kb) <= stored_pair_bound(kb, wl.dtype)).all(), rk


def test_invalid_host_arguments_raise():
    from causal_streaming_decoding_amd import wedlm as W
    t = torch.zeros(16, dtype=torch.int32, device="cuda")
    u = torch.zeros(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(W.WedlmError):
        W.wedlm_window_reorder(1, 65, u, t, t, t, t, t, t)


@pytest.mark.parametrize("wl", [
    _variant(WL.QWEN3_8B_BS1, name="flags_nw4", B=3, V=2048, prefix=("uniform", 100, 900)),
    _variant(WL.QWEN25_7B_RAGGED, name="flags_rowparts", B=3, V=2048, prefix=("uniform", 100, 900)),
])
def test_cache_policy_flag_bitwise_same(wl):
    """The shared-pages flag only changes the cache hint of the page loads:
    outputs with and without it are bitwise equal (one 4-wave workgroup per
    work unit, and four row parts per work unit)."""
    from causal_streaming_decoding_amd import wedlm as W_
    from causal_streaming_decoding_amd.step import make_window_step, upload_step_inputs

    print(f"[parity] {wl.name}", flush=True)
    inp = make_step_inputs(wl)
    st, q, k, v, _, mpl = upload_step_inputs(wl, inp, "cuda:0")
    step = make_window_step(wl, inp, "cuda:0", mpl)
    step.reorder(st, None)
    outs = []
    for flags in (0, W_.WEDLM_ATTN_SHARED_PAGES):
        out = torch.empty_like(step.out_phys)
        W_.wedlm_window_attn_rope(step.dt, step.n_layers, step.B, step.W, step.Hq, step.Hkv,
                                  step.D, step.page_size, step.num_pages, step.max_pages, mpl,
                                  step.scale, step.theta, q, k, v, step.perm, step.pos,
                                  st.k_cache, st.v_cache, st.block_table, st.prefix_len, None,
                                  out, step.attn_ws, step.attn_ws_bytes, flags=flags)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
