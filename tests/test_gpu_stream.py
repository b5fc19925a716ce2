"""Streaming loop at the full 36-layer, BS=16 Qwen3-8B shape against the oracle (GPU).

The GPU runs every layer of every step; the oracle replays the same steps in
lockstep on host copies of the same inputs (each step's inputs are dropped
once both sides have used them, so the whole 256-step loop fits in memory).
Every step's reorder, entropies, argmax, selection, commit lengths, cache
slots and window state are compared; the attention output and the committed
cache rows are compared on sampled layers (the oracle tracks only those
layers' caches). A flagged near-tie decision takes the GPU's choice for that
comparison only; every slot of every selection is compared.
"""

import dataclasses
import os

import numpy as np
import pytest
import torch

import oracle
from causal_streaming_decoding_amd import layout
from causal_streaming_decoding_amd import workloads as WL
from causal_streaming_decoding_amd.decode_stats import decode_counters
from causal_streaming_decoding_amd.wedlm import COMMIT_BLOCK, COMMIT_STREAM
from causal_streaming_decoding_amd.step import make_window_step, upload_step_inputs
from causal_streaming_decoding_amd.synth import make_step_inputs, stream_step_inputs, to_f64

from .parity import ATTN_ATOL, ATTN_RTOL, ENTROPY_ATOL, stored_pair_bound, storage_rounding

pytestmark = pytest.mark.gpu


ORDER_KEYS = ("perm", "inv", "pos", "run_len")
# host threads for the oracle's entropy rows (the machine's CPU share)
WORKERS = min(16, len(os.sched_getaffinity(0)))


def _to_host_f32(t):
    """Exact float32 host copy of a bf16 / f32 device tensor (half the bytes of f64)."""
    return t.detach().cpu().to(torch.float32).numpy()


def _run_stream(wl, steps, sampled_layers, attend_steps, commit_rule="stream", fused_tail=False,
                attend_after_len=None, progress_every=0):
    """Run ``steps`` window steps on the GPU and in the oracle in lockstep.

    attend_steps: steps whose attention is compared on the sampled layers;
    attend_after_len: also the first step at which every sequence's prefix
    has reached that length (e.g. just after the first page crossing).
    """
    print(f"[stream] {wl.name} steps={steps} layers={sampled_layers} tau={wl.tau} "
          f"rule={commit_rule} fused_tail={fused_tail}", flush=True)
    dev = "cuda"
    inp = make_step_inputs(wl, steps=wl.steps)
    st, _, _, _, _, L0 = upload_step_inputs(wl, inp, dev)
    rule = {"stream": COMMIT_STREAM, "block": COMMIT_BLOCK}[commit_rule]
    step = make_window_step(wl, inp, dev, L0 + wl.W * steps, commit_rule=rule,
                            fused_tail=fused_tail)
    if fused_tail:
        # the first step's order; every later one is written by the previous tail
        step.reorder(st)
    gpu_log = []
    attended = []
    state = {"crossed": attend_after_len is None}

    def gpu_step(s):
        """Runs GPU step s; returns the host inputs of the oracle's step s."""
        q, k, v, logits = stream_step_inputs(wl, s, dev)
        mpl = L0 + wl.W * s
        rec_prefix_in = st.prefix_len.cpu().numpy()
        attend = s in attend_steps
        if not state["crossed"] and rec_prefix_in.min() >= attend_after_len:
            state["crossed"] = attend = True
        # the order a step attends with: before the call under the fused tail
        # (which leaves the next step's order behind), after it otherwise
        order = {key: getattr(step, key).cpu().numpy() for key in ORDER_KEYS}
        step.run(st, q, k, v, logits, max_prefix_len=mpl)
        torch.cuda.synchronize()
        rec = {key: getattr(step, key).cpu().numpy() for key in
               ORDER_KEYS + ("entropy", "argmax", "selected", "commit_len", "cache_slot")}
        if fused_tail:
            rec.update(order)
        rec["prefix_len_in"] = rec_prefix_in
        rec["tokens"] = st.tokens.cpu().numpy()
        rec["filled"] = st.filled.cpu().numpy()
        rec["prefix_len"] = st.prefix_len.cpu().numpy()
        if attend:
            rec["attn"] = {i: to_f64(step.out_phys[l]) for i, l in enumerate(sampled_layers)}
            attended.append((s, int(rec_prefix_in.min())))
        gpu_log.append(rec)
        return (_to_host_f32(q[sampled_layers]), _to_host_f32(k[sampled_layers]),
                _to_host_f32(v[sampled_layers]), _to_host_f32(logits))

    flags = [0]

    def compare(s, r):
        g = gpu_log[s]
        assert np.array_equal(g["perm"], r["perm"]), ("perm", s)
        # the reorder reports the commit rule's count (the raw run when streaming)
        expect_run = [oracle.commit_count(x, wl.W, commit_rule) for x in r["run"]]
        assert np.array_equal(g["run_len"], expect_run), ("run", s)
        assert (np.abs(g["entropy"] - r["entropy"]) <= ENTROPY_ATOL).all(), ("entropy", s)
        assert np.array_equal(g["argmax"], r["argmax"]), ("argmax", s)
        flags[0] += len(r["flags"])
        # every slot: a flagged decision already took the GPU's choice
        assert np.array_equal(g["selected"].astype(bool), r["selected"]), ("sel", s)
        assert np.array_equal(g["commit_len"], r["commit_len"]), ("commit_len", s)
        assert np.array_equal(g["cache_slot"], r["cache_slot"]), ("cache_slot", s)
        assert np.array_equal(g["tokens"], r["tokens"]), ("tokens", s)
        assert np.array_equal(g["filled"].astype(bool), r["filled"]), ("filled", s)
        assert np.array_equal(g["prefix_len"], r["prefix_len"]), ("prefix_len", s)
        if "attn" in g:
            for i in g["attn"]:
                err = np.abs(g["attn"][i] - r["attn_out_phys"][i])
                ok = err <= ATTN_ATOL + ATTN_RTOL * np.abs(r["attn_out_phys"][i])
                assert ok.all(), ("attn", s, i, float(err.max()))
            del g["attn"]
        # keep only what the decoding counters need
        ref_log.append({"prefix_len_in": r["prefix_len_in"], "selected": r["selected"],
                        "commit_len": r["commit_len"]})
        if progress_every and (s + 1) % progress_every == 0:
            print(f"[stream] {wl.name}: step {s + 1}/{steps} ok, prefix "
                  f"{int(r['prefix_len'].min())}..{int(r['prefix_len'].max())}", flush=True)

    ref_log = []
    kc = [[np.asarray(x, np.float64) for x in inp["k_cache"][l]] for l in sampled_layers]
    vc = [[np.asarray(x, np.float64) for x in inp["v_cache"][l]] for l in sampled_layers]
    init_len = np.asarray(inp["prefix_len"]).copy()
    del inp["k_cache"], inp["v_cache"]

    def attend(s):
        return range(len(sampled_layers)) if "attn" in gpu_log[s] else []

    out = oracle.stream_loop(
        inp["filled"], inp["tokens"], inp["prefix_len"], kc, vc, inp["block_table"], steps,
        gpu_step, wl.theta, wl.lam, wl.tau, wl.page_size, wl.min_fill, wl.mask_id,
        attend=attend, track_layers=range(len(sampled_layers)),
        adopt_selected=lambda s, b: gpu_log[s]["selected"][b].astype(bool),
        on_step=compare, store=storage_rounding(wl.dtype), commit_rule=commit_rule,
        workers=WORKERS)
    del kc, vc
    assert state["crossed"], "no step reached the requested prefix length"

    # committed rows of the sampled layers, read back from the pages
    final_len = st.prefix_len.cpu().numpy()
    for i, l in enumerate(sampled_layers):
        for b in range(wl.B):
            L = int(init_len[b])
            n = int(final_len[b]) - L
            kr, vr = layout.read_rows(st.k_cache, st.v_cache, l, st.block_table[b].cpu(), L, n)
            kr, vr = to_f64(kr), to_f64(vr)
            ref_k = out["caches"][i][0][b][L:]
            ref_v = out["caches"][i][1][b][L:]
            assert kr.shape == ref_k.shape
            # the oracle's cache holds its rows as stored (rounded once), like the GPU's
            assert (np.abs(kr - ref_k) <= stored_pair_bound(ref_k, wl.dtype)).all(), ("cache k", i, b)
            assert np.array_equal(vr, ref_v), ("cache v", i, b)
    total = int(sum(g["commit_len"].sum() for g in gpu_log))
    longest = int(max(g["commit_len"].max() for g in gpu_log))
    # the decoding counters of the two runs agree exactly
    cg = decode_counters([{"prefix_len_in": g["prefix_len_in"], "selected": g["selected"],
                           "commit_len": g["commit_len"]} for g in gpu_log], wl.W)
    cr = decode_counters(ref_log, wl.W)
    assert cg == cr, (cg, cr)
    print(f"[stream] {wl.name}: {steps} steps ok, committed {total}, longest commit {longest}, "
          f"flags {flags[0]}, attention checked at (step, min prefix) {attended}, "
          f"p_cache {cg['p_cache']}, tokens/forward {cg['tokens_per_forward']:.3f}", flush=True)
    return total, longest, cg


@pytest.mark.timeout(900)
def test_stream_full_shape_all_steps_fused_tail():
    # the loop bench.py times: 36 layers, 16 sequences, vocabulary 151936, all
    # 256 steps with the fused tail; attention on three layers at the first
    # steps, just after every sequence's first page crossing (prefix 1040),
    # spread over the run and at the last step
    wl = WL.QWEN3_8B_STREAM
    _run_stream(wl, steps=wl.steps, sampled_layers=[0, 17, 35],
                attend_steps={0, 1, 64, 128, 192, wl.steps - 1}, fused_tail=True,
                attend_after_len=wl.prefix[1] + wl.page_size, progress_every=32)


def test_stream_full_shape_separate_tail_first_steps():
    # the same loop with the three separate calls after the entropy pass
    _run_stream(WL.QWEN3_8B_STREAM, steps=12, sampled_layers=[0, 17, 35], attend_steps={0, 5, 11})


def test_stream_low_entropy_multi_commit():
    # big spikes make the threshold fire, so runs longer than one token are committed
    wl = dataclasses.replace(WL.QWEN3_8B_STREAM, name="stream_low_entropy", n_layers=4, B=8,
                             V=30000, spike=("prob", 0.9, 16.0, 20.0))
    _, longest, _ = _run_stream(wl, steps=24, sampled_layers=[0, 3], attend_steps={3, 23})
    assert longest > 1  # multi-token commits happened


def test_stream_one_by_one_mode():
    # threshold None of the released engine: tau = -inf, one fill per step
    wl = dataclasses.replace(WL.QWEN3_8B_STREAM, name="stream_one_by_one", n_layers=4, B=8,
                             tau=float("-inf"))
    _, longest, c = _run_stream(wl, steps=24, sampled_layers=[1], attend_steps={5})
    assert c["predictions_per_forward"] <= 1.0


def test_stream_block_rule():
    # stop-and-wait on the same kernels: whole windows are cached, W + 1 steps apart
    wl = dataclasses.replace(WL.QWEN3_8B_STREAM, name="stream_block", n_layers=4, B=8,
                             tau=float("-inf"))
    _, longest, c = _run_stream(wl, steps=3 * (wl.W + 1), sampled_layers=[0, 2],
                                attend_steps={0, wl.W, wl.W + 1}, commit_rule="block")
    assert longest == wl.W
    assert set(c["delay_histogram"]) == set(range(1, wl.W + 1))


def test_stream_block_rule_low_entropy():
    # threshold fills several slots per step: a window completes sooner
    wl = dataclasses.replace(WL.QWEN3_8B_STREAM, name="stream_block_low_entropy", n_layers=4,
                             B=8, V=30000, spike=("prob", 0.9, 16.0, 20.0))
    _, longest, c = _run_stream(wl, steps=24, sampled_layers=[3], attend_steps={7},
                                commit_rule="block")
    assert longest == wl.W


def test_stream_fused_tail():
    # selection + state commit + next reorder as one call, against the oracle
    wl = dataclasses.replace(WL.QWEN3_8B_STREAM, name="stream_fused_tail", n_layers=4, B=8,
                             V=30000, spike=("prob", 0.9, 16.0, 20.0))
    _, longest, _ = _run_stream(wl, steps=24, sampled_layers=[0, 3], attend_steps={0, 1, 23},
                                fused_tail=True)
    assert longest > 1


def test_stream_fused_tail_block_rule():
    wl = dataclasses.replace(WL.QWEN3_8B_STREAM, name="stream_fused_tail_block", n_layers=4,
                             B=8, tau=float("-inf"))
    _, longest, _ = _run_stream(wl, steps=2 * (wl.W + 1), sampled_layers=[1],
                                attend_steps={wl.W}, commit_rule="block", fused_tail=True)
    assert longest == wl.W
