"""The fused-tail step with the entropy chunk pass beside the attention (GPU).

Two forms: wedlm_entropy_partials on a side stream beside
wedlm_window_attn_rope, and wedlm_window_attn_rope_entropy, whose launch
carries the chunk blocks after the attention's workgroups; in both,
wedlm_select_commit_reorder_partials merges afterwards. The one-launch form
also runs with the merge of split attention partials deferred to the tail's
launch (WEDLM_ATTN_DEFER_COMBINE + wedlm_select_commit_reorder_combine). The
computations are those of the one-stream step, so every output of every step
of a chained run must be bitwise the same. The chain checks the ordering
between a step's tail and the next step's chunk pass, which write and read the
same workspace.
"""

import dataclasses

import pytest
import torch

from causal_streaming_decoding_amd import workloads as WL
from causal_streaming_decoding_amd.step import make_window_step, upload_step_inputs
from causal_streaming_decoding_amd.synth import make_step_inputs, stream_step_inputs

pytestmark = pytest.mark.gpu

OUTPUTS = ("out_phys", "entropy", "score", "argmax", "selected", "commit_len", "cache_slot",
           "perm", "inv", "pos", "n_obs", "run_len")


def _chain(wl, steps, overlap, fuse=False, defer=False):
    inp = make_step_inputs(wl, steps=steps)
    st, _, _, _, _, L0 = upload_step_inputs(wl, inp, "cuda")
    step = make_window_step(wl, inp, "cuda", L0 + wl.W * steps, fused_tail=True)
    if overlap:
        step.set_overlap(torch.cuda.Stream())
    step.fuse_entropy = fuse
    step.defer_combine = defer
    log = []
    for s in range(steps):
        q, k, v, logits = stream_step_inputs(wl, s, "cuda")
        step.run(st, q, k, v, logits, max_prefix_len=L0 + wl.W * s)
        torch.cuda.synchronize()
        rec = {key: getattr(step, key).clone() for key in OUTPUTS}
        rec.update(tokens=st.tokens.clone(), filled=st.filled.clone(),
                   prefix_len=st.prefix_len.clone())
        log.append(rec)
    return log, st


@pytest.mark.parametrize("wl", [
    dataclasses.replace(WL.QWEN3_8B_STREAM, name="overlap_stream", n_layers=4, B=8, V=30000,
                        spike=("prob", 0.9, 16.0, 20.0), steps=12),
    dataclasses.replace(WL.QWEN3_8B_STREAM, name="overlap_bs1_split", n_layers=1, B=1, V=151936,
                        prefix=("fixed", 2048), steps=6),
    # row parts, ragged split plan, an odd vocabulary (element-wise chunk path)
    dataclasses.replace(WL.QWEN25_7B_RAGGED, name="overlap_gqa7_odd_vocab", B=3, V=5001,
                        fill=("none",), spike=("prob", 0.9, 16.0, 20.0), steps=5),
    # 100 sequences: the tail launch's 100 per-sequence wavefronts before the
    # merge workgroups, a split plan scanning sequences in wavefront-wide chunks
    dataclasses.replace(WL.QWEN3_8B_BS1, name="overlap_b100_split", B=100, V=4096,
                        prefix=("uniform", 16, 600), steps=3),
], ids=lambda w: w.name)
def test_overlapped_step_bitwise_equal(wl):
    print(f"[overlap] {wl.name}: {wl.steps} chained steps", flush=True)
    one, st1 = _chain(wl, wl.steps, overlap=False)
    for form, kw in (("two streams", dict(overlap=True)),
                     ("one launch", dict(overlap=False, fuse=True)),
                     ("one launch, merge in the tail", dict(overlap=False, fuse=True, defer=True))):
        two, st2 = _chain(wl, wl.steps, **kw)
        for s, (a, b) in enumerate(zip(one, two)):
            for key in a:
                assert torch.equal(a[key], b[key]), (wl.name, form, s, key)
        assert torch.equal(st1.k_cache, st2.k_cache) and torch.equal(st1.v_cache, st2.v_cache)
        print(f"[overlap] {wl.name} ({form}): every step bitwise equal", flush=True)
