"""Host mirror of the attention kernel's key-range split plan for ragged
batches, checked against the properties the plan must have.

In split mode each (layer, kv head) column has S workgroups. Sequence b's work
is u_b = ceil(L_b / 16) prefix pages + ceil(W / 16) window chunks; with a split
size of K units it takes ceil(u_b / K) consecutive workgroups, split s covering
pages [s K, (s+1) K), the last split also the window. K is the smallest value
(>= min_pages) whose split counts fit in S, searched between ceil(P / S) and
ceil((P - B) / (S - B)). The GPU parity cases run the kernel's own plan; this
test pins the arithmetic: every page covered exactly once, every window once,
no workgroup over K units, no more than S workgroups, and the upper end of the
search interval always feasible.
"""

import numpy as np
import pytest

PAGE = 16


def plan(lengths, W, S, min_pages, max_prefix):
    B = len(lengths)
    assert S > B
    pages = [(min(max(int(L), 0), max_prefix) + PAGE - 1) // PAGE for L in lengths]
    units = [p + (W + PAGE - 1) // PAGE for p in pages]
    P = sum(units)

    def fits(K):
        return sum((u + K - 1) // K for u in units) <= S

    lo = max(min_pages, (P + S - 1) // S)
    hi = max(lo, (P - B + (S - B) - 1) // (S - B))
    assert fits(hi), "upper end of the search interval must fit"
    while lo < hi:
        mid = (lo + hi) // 2
        if fits(mid):
            hi = mid
        else:
            lo = mid + 1
    K = lo
    counts = [(u + K - 1) // K for u in units]
    # workgroup j of the column -> (sequence, split), as the kernel's scan finds it
    assignment = {}
    first = 0
    for b, n in enumerate(counts):
        for s in range(n):
            assignment[first + s] = (b, s, n)
        first += n
    return K, pages, assignment


@pytest.mark.parametrize("seed", range(40))
def test_split_plan_covers_each_page_once(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 150))
    max_prefix = int(rng.integers(0, 6000))
    lengths = rng.integers(-2, max_prefix + 30, size=B)
    W = int(rng.integers(1, 65))
    min_pages = int(rng.choice([4, 6, 8]))
    S = B + int(rng.integers(1, 1300))
    K, pages, assignment = plan(lengths, W, S, min_pages, max_prefix)
    assert K >= min_pages
    assert len(assignment) <= S and all(0 <= j < S for j in assignment)
    cover = [np.zeros(p, dtype=np.int64) for p in pages]
    windows = np.zeros(B, dtype=np.int64)
    for b, s, n in assignment.values():
        lo = min(pages[b], s * K)
        hi = min(pages[b], lo + K)
        cover[b][lo:hi] += 1
        work = hi - lo
        if s == n - 1:
            windows[b] += 1
            work += (W + PAGE - 1) // PAGE
        assert work <= K
    for b in range(B):
        assert (cover[b] == 1).all()
    assert (windows == 1).all()


def test_split_plan_balances_a_ragged_batch():
    # 16 sequences with prefixes 512..4096, W = 32, 64 workgroups per column:
    # the longest sequence is spread over several splits of about the mean size
    rng = np.random.default_rng(0)
    lengths = rng.integers(512, 4097, size=16)
    K, pages, assignment = plan(lengths, 32, 64, 8, 4096)
    mean_units = (sum(pages) + 16 * 2) / 64
    assert K <= 1.5 * mean_units
    assert max(p for p in pages) > 2 * K  # the long ones are split
