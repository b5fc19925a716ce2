"""One window step captured as a HIP graph, replayed against the eager step (GPU).

The graph holds the step's kernel launches only (reorder, attention with fused
RoPE and append, the split combine where the key ranges are split, the
entropy pass and the fused tail). Each replay runs on the window state the
buffers hold, so the state is restored eagerly before every replay, with
other eager GPU work and synchronisations in between; every replay's outputs
must be bitwise those of the eager step on the same state.
"""

import dataclasses

import numpy as np
import pytest
import torch

from causal_streaming_decoding_amd import workloads as WL
from causal_streaming_decoding_amd.step import make_window_step, upload_step_inputs
from causal_streaming_decoding_amd.synth import make_step_inputs

pytestmark = pytest.mark.gpu

OUTPUTS = ("out_phys", "entropy", "score", "argmax", "selected", "commit_len", "cache_slot",
           "perm", "inv", "pos", "n_obs", "run_len")


def _snapshot_outputs(step, st):
    o = {k: getattr(step, k).clone() for k in OUTPUTS}
    o.update(tokens=st.tokens.clone(), filled=st.filled.clone(), prefix_len=st.prefix_len.clone(),
             k_cache=st.k_cache.clone(), v_cache=st.v_cache.clone())
    return o


def _poison_outputs(step):
    # replays must write every output: clear them to values no step produces
    for k in OUTPUTS:
        t = getattr(step, k)
        if t.is_floating_point():
            t.fill_(float("nan"))
        else:
            t.fill_(253 if t.dtype == torch.uint8 else -3)


@pytest.mark.parametrize("wl", [
    # key ranges split across workgroups: the combine kernel is in the graph
    dataclasses.replace(WL.QWEN3_8B_BS1, name="graph_bs1", B=2, V=8192),
    # 224 rows in four row parts, ragged split plan
    dataclasses.replace(WL.QWEN25_7B_RAGGED, name="graph_gqa7", B=3, V=4096),
    # many groups, no split; several layers
    dataclasses.replace(WL.QWEN3_8B_STREAM, name="graph_layers", n_layers=4, B=8, V=4096,
                        fill=("frac", 0.0, 1.0), steps=1),
    WL.TINY_FP32,
], ids=lambda w: w.name)
def test_step_graph_replays_match_eager(wl):
    print(f"[graph] {wl.name}", flush=True)
    inp = make_step_inputs(wl)
    st, q, k, v, logits, mpl = upload_step_inputs(wl, inp, "cuda")
    step = make_window_step(wl, inp, "cuda", mpl, fused_tail=True)
    snap = st.snapshot()
    caches = (st.k_cache.clone(), st.v_cache.clone())
    step.run(st, q, k, v, logits)
    torch.cuda.synchronize()
    ref = _snapshot_outputs(step, st)

    st.restore(snap)
    g = step.capture(st, q, k, v, logits)
    assert st.ordered_by is None  # capturing ran nothing
    scratch = torch.randn(1 << 20, device="cuda")
    for r in range(3):
        st.restore(snap)
        st.k_cache.copy_(caches[0])
        st.v_cache.copy_(caches[1])
        _poison_outputs(step)
        scratch.mul_(1.0001).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot_outputs(step, st)
        for key in ref:
            a, b = got[key], ref[key]
            same = torch.equal(a, b) if not a.is_floating_point() else bool(
                ((a == b) | (torch.isnan(a) & torch.isnan(b))).all())
            assert same, (wl.name, r, key)
    print(f"[graph] {wl.name}: 3 replays bitwise equal to the eager step", flush=True)
