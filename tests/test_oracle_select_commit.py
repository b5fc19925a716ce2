"""Pins for the oracle's selection, commit and refill (CPU).

Hand-worked cases (tests/golden/select_commit_cases.json, each with its
derivation) and conservation laws of the streaming loop. The floor rule
(fill the lowest-score mask slot when nothing clears the threshold) is a
reading of the pages, so its parity with the pages is unpinned; the cases pin
the oracle to that stated reading.
"""

import json
import os

import numpy as np
import pytest

from oracle import commit_and_refill, select_slots, topological_reorder
from oracle import rope_rotate, stream_loop

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "select_commit_cases.json")


def _cases():
    with open(GOLDEN) as fh:
        data = json.load(fh)
    return data["page_size"], data["mask_id"], data["cases"]


PAGE, MASK, CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_golden_case(case):
    tau = float("-inf") if case["tau"] == "-inf" else case["tau"]
    filled = np.array(case["filled"], bool)
    s = select_slots(case["entropy"], filled, case["lam"], tau, case["min_fill"])
    e = case["expect"]
    assert s["selected"].astype(int).tolist() == e["selected"]
    assert s["fallback"] == e["fallback"]
    r = topological_reorder(filled, case["prefix_len"])
    assert r["run"] == e["run"]
    c = commit_and_refill(case["tokens"], filled, case["prefix_len"], r["run"], s["selected"],
                          case["argmax"], case["block_table"], PAGE, MASK)
    assert c["commit_len"] == e["commit_len"]
    assert c["committed"].tolist() == e["committed"]
    assert c["cache_slot"].tolist() == e["cache_slot"]
    assert c["filled"].astype(int).tolist() == e["filled"]
    assert c["tokens"].tolist() == e["tokens"]
    assert c["prefix_len"] == e["prefix_len"]


def test_tie_flags():
    s = select_slots([1.0, 0.5], [False, False], 0.5, 1.0, 1)
    kinds = sorted(s["flags"])
    assert ("threshold", 0) in kinds and ("threshold", 1) in kinds and ("fallback", 1) in kinds
    s = select_slots([0.2, 3.0], [False, False], 0.1, 1.0, 1)
    assert s["flags"] == []


def test_scores_and_decisions_are_float64():
    # 1 - 2^-40 clears tau = 1 in float64; the float32 rounding of the same
    # score would be exactly 1.0 and would not (strict comparison)
    h = 1.0 - 2.0 ** -40
    s = select_slots([h, 9.0], [False, False], 0.0, 1.0, 1)
    assert s["score"].dtype == np.float64 and s["score"][0] == h
    assert s["selected"].tolist() == [True, False] and not s["fallback"]
    assert ("threshold", 0) in s["flags"]


def test_adopt_takes_only_flagged_threshold_decisions():
    # slot 0's score is within 1e-4 of tau: flagged, so the other side's
    # decision for it is taken; slot 1 is far from every boundary
    H = [1.00005, 5.0]
    own = select_slots(H, [False, False], 0.0, 1.0, 1)
    assert own["selected"].tolist() == [True, False] and own["fallback"]  # floor rule
    s = select_slots(H, [False, False], 0.0, 1.0, 1, adopt=[True, False])
    assert s["selected"].tolist() == [True, False] and not s["fallback"]  # adopted threshold
    # an unflagged difference is not adopted: the caller's slot-by-slot
    # comparison will see it
    s = select_slots(H, [False, False], 0.0, 1.0, 1, adopt=[False, True])
    assert s["selected"].tolist() == [True, False]
    # far from the threshold nothing is adopted
    s = select_slots([0.2, 3.0], [False, False], 0.1, 1.0, 1, adopt=[False, True])
    assert s["selected"].tolist() == [True, False] and s["flags"] == []


def test_adopt_floor_rule_tie():
    # floor rule: slots 1 and 2 score 3.0 and 3.00005 (a near tie), slot 3 far above
    H = [0.0, 2.9, 2.80005, 9.0]
    f = [True, False, False, False]
    own = select_slots(H, f, 0.1, 1.0, 1)
    assert own["selected"].tolist() == [False, True, False, False]
    assert own["flags"] == [("fallback", 2)]
    s = select_slots(H, f, 0.1, 1.0, 1, adopt=[False, False, True, False])
    assert s["selected"].tolist() == [False, False, True, False]
    # a pick outside the tied set, or two picks, leave the oracle's own choice
    for other in ([False, False, False, True], [False, True, True, False]):
        s = select_slots(H, f, 0.1, 1.0, 1, adopt=other)
        assert s["selected"].tolist() == [False, True, False, False]


def test_commit_rejects_a_wrong_run():
    with pytest.raises(ValueError):
        commit_and_refill([1, -1], [True, False], 0, 2, [False, False], [0, 0], [0], 16)
    with pytest.raises(ValueError):
        commit_and_refill([1, 2], [True, True], 0, 1, [False, False], [0, 0], [0], 16)


def _small_stream(seed, steps, nl=2, B=3, Hq=4, Hkv=2, D=16, W=8, V=64, L0=5, theta=1e4):
    rng = np.random.default_rng(seed)
    k_raw = [[rng.standard_normal((L0, Hkv, D)) for _ in range(B)] for _ in range(nl)]
    v_pre = [[rng.standard_normal((L0, Hkv, D)) for _ in range(B)] for _ in range(nl)]
    k_cache = [[rope_rotate(k_raw[l][b], np.arange(L0)[:, None], theta) for b in range(B)]
               for l in range(nl)]
    per_step = []
    for _ in range(steps):
        q = rng.standard_normal((nl, B, W, Hq, D))
        k = rng.standard_normal((nl, B, W, Hkv, D))
        v = rng.standard_normal((nl, B, W, Hkv, D))
        logits = rng.normal(0, 2, size=(B, W, V))
        hit = rng.random((B, W)) < 0.7
        tok = rng.integers(0, V, size=(B, W))
        logits[hit, tok[hit]] += rng.uniform(6, 16, size=int(hit.sum()))
        per_step.append((q, k, v, logits))
    pages = (L0 + W * steps + PAGE - 1) // PAGE
    table = np.array([rng.permutation(1000)[:pages] for _ in range(B)])
    return dict(k_cache=k_cache, v_cache=v_pre, per_step=per_step, table=table, L0=L0, W=W, B=B,
                theta=theta)


def test_stream_loop_conservation_laws():
    steps = 40
    d = _small_stream(0, steps)
    B, W, L0 = d["B"], d["W"], d["L0"]
    log = []

    def on_step(s, r):
        log.append(r)

    out = stream_loop(np.zeros((B, W), bool), np.full((B, W), -1), np.full(B, L0), d["k_cache"],
                      d["v_cache"], d["table"], steps, lambda s: d["per_step"][s], d["theta"],
                      lam=0.1, tau=1.5, page_size=PAGE, attend=lambda s: [0, 1] if s % 7 == 0 else [],
                      track_layers=[0, 1], on_step=on_step)
    total = out["commit_len"].sum(axis=0)
    assert np.array_equal(out["prefix_len"] - L0, total)              # sum of c = growth of L
    assert out["total_committed"] == int(total.sum())
    # a decoded stream per sequence: every committed token is the argmax chosen
    # when its slot was filled, and committed positions are contiguous
    chosen = [dict() for _ in range(B)]
    committed_stream = [[] for _ in range(B)]
    appended = {(layer, b): [] for layer in (0, 1) for b in range(B)}
    for s, r in enumerate(log):
        q, k, v, _ = d["per_step"][s]
        for layer in (0, 1):
            for b in range(B):
                L = int(r["prefix_len_in"][b])
                for j in range(int(r["commit_len"][b])):
                    appended[(layer, b)].append(rope_rotate(k[layer, b, j], L + j, d["theta"]))
    for r in log:
        for b in range(B):
            L = r["pos"][b][r["inv"][b][0]]                          # logical position of slot 0
            c = int(r["commit_len"][b])
            assert c <= r["n_obs"][b] and c <= W
            assert c == W or not r["filled_in"][b][c]                  # slot c is a mask
            for j in range(c):
                committed_stream[b].append((L + j, int(r["committed"][b][j])))
            for i in np.flatnonzero(r["selected"][b]):
                chosen[b][int(L + i)] = int(r["argmax"][b][i])
            if c:
                slots = r["cache_slot"][b][:c]
                assert len(set(slots.tolist())) == c
    for b in range(B):
        positions = [p for p, _ in committed_stream[b]]
        assert positions == list(range(L0, L0 + len(positions)))
        for p, tok in committed_stream[b]:
            assert chosen[b][p] == tok
    # tracked caches grew by exactly the committed rows, each rotated at its position
    for layer in (0, 1):
        for b in range(B):
            kc = out["caches"][layer][0][b]
            assert kc.shape[0] == out["prefix_len"][b]
            rows = appended[(layer, b)]
            if rows:
                assert np.array_equal(kc[L0:], np.stack(rows))


def test_stream_loop_progresses_with_floor_rule():
    # with tau = -inf only the floor rule fills; every step fills exactly one mask slot
    steps = 30
    d = _small_stream(1, steps)
    B, W, L0 = d["B"], d["W"], d["L0"]
    fills = []
    out = stream_loop(np.zeros((B, W), bool), np.full((B, W), -1), np.full(B, L0), d["k_cache"],
                      d["v_cache"], d["table"], steps, lambda s: d["per_step"][s], d["theta"],
                      lam=0.1, tau=float("-inf"), page_size=PAGE,
                      on_step=lambda s, r: fills.append(r["selected"].sum(axis=1)))
    assert all((f == 1).all() for f in fills)
    # tokens in = tokens out: the window holds what was filled and not yet committed
    commits = out["commit_len"].sum(axis=0)
    assert np.array_equal(out["filled"].sum(axis=1), steps - commits)
    assert (commits >= steps - W).all()


def test_block_rule_commits_only_whole_windows():
    from oracle import commit_count
    assert [commit_count(r, 4, "stream") for r in range(5)] == [0, 1, 2, 3, 4]
    assert [commit_count(r, 4, "block") for r in range(5)] == [0, 0, 0, 0, 4]
    with pytest.raises(ValueError):
        commit_count(1, 4, "other")
    table = np.arange(8)
    # three of four slots filled: nothing is cached, the fills stay in the window
    c = commit_and_refill([5, 6, 7, -1], [1, 1, 1, 0], 16, 3, [0, 0, 0, 1], [0, 0, 0, 9], table,
                          PAGE, rule="block")
    assert c["commit_len"] == 0 and c["prefix_len"] == 16
    assert c["filled"].tolist() == [True] * 4 and c["tokens"].tolist() == [5, 6, 7, 9]
    assert (c["cache_slot"] == -1).all()
    # a full window: cached at once, replaced by four masks
    c = commit_and_refill([5, 6, 7, 9], [1, 1, 1, 1], 16, 4, [0, 0, 0, 0], [0, 0, 0, 0], table,
                          PAGE, rule="block")
    assert c["commit_len"] == 4 and c["prefix_len"] == 20
    assert c["committed"].tolist() == [5, 6, 7, 9]
    assert not c["filled"].any() and (c["tokens"] == -1).all()
    assert c["cache_slot"].tolist() == [16 + j for j in range(4)]  # page 1 of an identity table


def test_stream_loop_block_rule():
    # stop-and-wait: every commit is 0 or W, and with one fill per step (tau = -inf)
    # a window is cached every W steps
    steps = 3 * 8
    d = _small_stream(2, steps)
    B, W, L0 = d["B"], d["W"], d["L0"]
    out = stream_loop(np.zeros((B, W), bool), np.full((B, W), -1), np.full(B, L0), d["k_cache"],
                      d["v_cache"], d["table"], steps, lambda s: d["per_step"][s], d["theta"],
                      lam=0.1, tau=float("-inf"), page_size=PAGE, commit_rule="block")
    c = out["commit_len"]
    assert set(np.unique(c).tolist()) <= {0, W}
    # fills at steps 0..W-1 complete the first window; the step whose forward
    # sees it full commits it and has no mask left to predict (the pipeline
    # bubble of block decoding), so windows are cached every W + 1 steps
    commit_steps = [s for s in range(steps) if s >= W and (s - W) % (W + 1) == 0]
    expect = np.zeros_like(c)
    expect[commit_steps] = W
    assert np.array_equal(c, expect)
    assert np.array_equal(out["prefix_len"], np.full(B, L0 + W * len(commit_steps)))
