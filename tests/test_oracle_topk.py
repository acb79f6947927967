"""Pins for the oracle's top-k: brute force by Python's sort on
(-score, position) tuples, the k >= n_vis case, and the pages' worked
example of the fused lookup."""
import numpy as np

from oracle.topk import topk_lookup, topk_positions
from tests.golden.load import load


def _brute(scores, n_vis, k):
    pairs = sorted((-float(scores[s]), s) for s in range(n_vis))
    return [s for _, s in pairs[:k]]


def test_topk_matches_sorted_tuples_with_many_ties():
    rng = np.random.default_rng(7)
    for trial in range(50):
        L = int(rng.integers(1, 300))
        n_vis = int(rng.integers(1, L + 1))
        k = int(rng.integers(1, 350))
        scores = rng.integers(0, 12, L).astype(np.float64)   # dense ties
        got = topk_positions(scores, n_vis, k).tolist()
        assert got == _brute(scores, n_vis, k), (trial, L, n_vis, k)


def test_topk_float_scores_and_negative_values():
    rng = np.random.default_rng(8)
    scores = rng.standard_normal(500).astype(np.float32).astype(np.float64)
    scores[::7] = scores[3]                                  # planted ties
    got = topk_positions(scores, 480, 64).tolist()
    assert got == _brute(scores, 480, 64)


def test_k_at_least_n_vis_selects_every_visible_position():
    rng = np.random.default_rng(9)
    scores = rng.integers(0, 5, 40).astype(np.float64)
    got = topk_positions(scores, 33, 100)
    assert sorted(got.tolist()) == list(range(33))
    assert got.tolist() == _brute(scores, 33, 100)


def test_lim_worked_example():
    g = load("lim_example.txt")
    L = g["ctx_len"]
    cache_slots = np.array(g["cache_slots"], np.int32)
    # Any scores that rank 8, 4, 17 first; 18 ties with 17 and loses on the
    # lower-position rule.
    scores = np.zeros((1, L))
    scores[0, 8], scores[0, 4], scores[0, 17], scores[0, 18] = 30, 20, 10, 10
    sel_pos, sel_slot, n_sel = topk_lookup(scores, [L], g["topk"], cache_slots)
    assert sel_pos[0].tolist() == g["top_positions"]
    assert sel_slot[0].tolist() == g["top_slots"]
    assert n_sel.tolist() == [3]
    misses = sorted(p for p, s in zip(sel_pos[0], sel_slot[0]) if s < 0)
    assert misses == g["misses"]
    i = sel_pos[0].tolist().index(g["hit_position"])
    assert sel_slot[0, i] == g["hit_slot"]


def test_padding_beyond_n_sel():
    scores = np.arange(10, dtype=np.float64)[None, :]
    sel_pos, sel_slot, n_sel = topk_lookup(scores, [4], 6, np.full(10, -1))
    assert n_sel[0] == 4
    assert sel_pos[0].tolist() == [3, 2, 1, 0, -1, -1]
    assert sel_slot[0].tolist() == [-1] * 6
