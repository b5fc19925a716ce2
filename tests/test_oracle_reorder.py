"""Pins for the oracle's topological reorder (CPU).

The reorder is pinned by exhaustive enumeration against an independent rank
formula: a filled slot's physical index is the number of filled slots before
it; a mask slot's is n_obs plus the number of masks before it (hyper.ai
summary of WeDLM, "Method": filled tokens move to the front, masks to the end,
logical positions kept).
"""

import itertools

import numpy as np
import pytest

from oracle import topological_reorder, visible_mask


def rank_formula(filled, L):
    f = np.asarray(filled, dtype=np.int64)
    W = f.size
    n_obs = int(f.sum())
    filled_before = np.concatenate([[0], np.cumsum(f)[:-1]])
    masks_before = np.concatenate([[0], np.cumsum(1 - f)[:-1]])
    phys = np.where(f == 1, filled_before, n_obs + masks_before)
    perm = np.empty(W, np.int64)
    perm[phys] = np.arange(W)
    # leading run: index of the first zero, or W
    zeros = np.flatnonzero(f == 0)
    run = int(zeros[0]) if zeros.size else W
    return phys, perm, L + perm, n_obs, run


@pytest.mark.parametrize("W", range(1, 9))
def test_exhaustive_against_rank_formula(W):
    L = 40
    for bits in itertools.product([False, True], repeat=W):
        r = topological_reorder(bits, L)
        phys, perm, pos, n_obs, run = rank_formula(bits, L)
        assert np.array_equal(r["inv"], phys)
        assert np.array_equal(r["perm"], perm)
        assert np.array_equal(r["pos"], pos)
        assert r["n_obs"] == n_obs
        assert r["run"] == run


def test_properties_random_wide_windows():
    rng = np.random.default_rng(1)
    for _ in range(300):
        W = int(rng.integers(1, 65))
        f = rng.random(W) < rng.random()
        L = int(rng.integers(0, 5000))
        r = topological_reorder(f, L)
        perm, inv = r["perm"], r["inv"]
        assert sorted(perm.tolist()) == list(range(W))          # bijection
        assert np.array_equal(perm[inv], np.arange(W))          # inverse
        n = r["n_obs"]
        assert f[perm[:n]].all() and not f[perm[n:]].any()      # filled first
        assert np.all(np.diff(perm[:n]) > 0) and np.all(np.diff(perm[n:]) > 0)  # stable
        assert np.array_equal(r["pos"] - L, perm)               # logical positions kept
        assert f[: r["run"]].all() and (r["run"] == W or not f[r["run"]])


def test_leading_run_rows_are_their_own_slots():
    # the committed run's physical rows are exactly its slots
    rng = np.random.default_rng(2)
    for _ in range(200):
        W = int(rng.integers(1, 33))
        f = rng.random(W) < 0.7
        r = topological_reorder(f, 0)
        c = r["run"]
        assert np.array_equal(r["perm"][:c], np.arange(c))


@pytest.mark.parametrize("W", range(1, 9))
def test_visibility_is_physical_causal_order(W):
    # Form M's slot-order visibility equals "physical index of key <= physical
    # index of query" computed from the reorder.
    for bits in itertools.product([False, True], repeat=W):
        inv = topological_reorder(bits, 0)["inv"]
        expect = inv[None, :] <= inv[:, None]
        assert np.array_equal(visible_mask(bits), expect)


def test_mask_slots_see_every_observed_slot():
    rng = np.random.default_rng(3)
    for _ in range(100):
        W = int(rng.integers(1, 33))
        f = rng.random(W) < 0.5
        vis = visible_mask(f)
        for i in np.flatnonzero(~f):
            assert vis[i, f].all()
        for i in np.flatnonzero(f):
            assert not vis[i, ~f].any()                 # observed never see masks
            assert np.array_equal(vis[i, f], np.flatnonzero(f) <= i)
