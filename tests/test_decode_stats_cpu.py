"""Decoding counters (tokens / predictions per forward, p_cache, commit delay) on
hand-built runs, and on oracle runs whose commit pattern is known (CPU)."""

import numpy as np

from causal_streaming_decoding_amd.decode_stats import decode_counters
from oracle import stream_loop

from .test_oracle_select_commit import PAGE, _small_stream


def _rec(L, sel, c):
    return {"prefix_len_in": np.array([L]), "selected": np.array([sel], bool),
            "commit_len": np.array([c])}


def test_hand_built_run():
    # W = 4. step 0 fills slot 0 (position 10); step 1 commits it (delay 1) and
    # fills slot 1 (position 11) and slot 3 (position 13); step 2 commits 11
    # (delay 1); step 3 fills slot 1 (position 13 - 11 = 2? no: L = 12, slot 1
    # is position 13 - already filled - so it fills slot 0, position 12);
    # step 4 commits 12 and 13 (delays 1 and 3).
    recs = [_rec(10, [1, 0, 0, 0], 0),
            _rec(10, [0, 1, 0, 1], 1),
            _rec(11, [0, 0, 0, 0], 1),
            _rec(12, [1, 0, 0, 0], 0),
            _rec(12, [0, 0, 0, 0], 2)]
    c = decode_counters(recs, 4)
    assert c["steps"] == 5 and c["sequences"] == 1
    assert c["committed"] == 4 and c["predicted"] == 4
    assert c["tokens_per_forward"] == 4 / 5 and c["predictions_per_forward"] == 4 / 5
    assert c["delay_histogram"] == {1: 3, 3: 1}
    assert c["p_cache"] == 3 / 4 and c["mean_commit_delay"] == 6 / 4


def test_tokens_filled_before_the_run_have_no_delay():
    recs = [_rec(0, [0, 0, 0, 0], 2), _rec(2, [0, 0, 0, 0], 0)]
    c = decode_counters(recs, 4)
    assert c["committed"] == 2 and c["p_cache"] is None and c["mean_commit_delay"] is None


def _oracle_records(rule, tau, steps=24, seed=3):
    d = _small_stream(seed, steps)
    B, W, L0 = d["B"], d["W"], d["L0"]
    recs = []
    stream_loop(np.zeros((B, W), bool), np.full((B, W), -1), np.full(B, L0), d["k_cache"],
                d["v_cache"], d["table"], steps, lambda s: d["per_step"][s], d["theta"], lam=0.1,
                tau=tau, page_size=PAGE, commit_rule=rule,
                on_step=lambda s, r: recs.append({"prefix_len_in": r["prefix_len_in"],
                                                  "selected": r["selected"],
                                                  "commit_len": r["commit_len"]}))
    return recs, B, W


def test_one_by_one_streaming_counts():
    # tau = -inf: exactly one fill in every step whose window still has a mask
    # slot (the lowest-score one, not necessarily the leftmost)
    recs, B, W = _oracle_records("stream", float("-inf"))
    c = decode_counters(recs, W)
    steps_with_fill = sum(int(np.asarray(r["selected"]).any(axis=1).sum()) for r in recs)
    assert c["predicted"] == steps_with_fill
    assert c["committed"] == sum(int(np.asarray(r["commit_len"]).sum()) for r in recs)
    # every committed token was filled during the run; delays are at least one step
    assert sum(c["delay_histogram"].values()) == c["committed"]
    assert min(c["delay_histogram"]) >= 1
    assert 0.0 < c["p_cache"] <= 1.0


def test_block_rule_delays():
    # stop-and-wait with one fill per step: the window's W fills are cached
    # together, W, W - 1, ..., 1 steps after they were made
    recs, B, W = _oracle_records("block", float("-inf"))
    c = decode_counters(recs, W)
    # a window is cached every W + 1 steps (the committing step predicts nothing)
    blocks = len([s for s in range(len(recs)) if s >= W and (s - W) % (W + 1) == 0])
    assert c["predictions_per_forward"] == (len(recs) - blocks) / len(recs)
    assert c["committed"] == B * W * blocks
    assert c["delay_histogram"] == {d: B * blocks for d in range(1, W + 1)}
    assert c["p_cache"] == 1 / W
