"""Offline replay of the hot pool under different eviction policies.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix (FlashOffloading analysis, decode ablation, first group,
and Fig. 8):
  * the per-layer, per-step top-2048 index sets of a run are recorded and
    replayed offline through a simulator on the same access sequence,
    changing only the eviction policy: Random, LRU, Score (evict tokens with
    low scores) and LIM (a score threshold plus a chunk scan);
  * the finding: capacity dominates and policy is secondary (8192 -> 16384
    slots cut misses by 43-49 %; at 16384 slots Score beats LIM by 18-20 %,
    and the gap narrows as capacity grows).

Readings where the pages are silent:
  * every policy keeps the pool's step: the misses are the union of the
    step's ways minus the residents; victims are free slots first, then
    residents outside the union chosen by the policy; one victim per miss,
    so the pool never shrinks after the fill;
  * the replay starts from the decode's first fill: the top-min(C, n_vis)
    positions of way 0 at step 0 (score descending, position ascending);
  * LRU: least recently used first, with recency = the last step whose
    union held the position and, within a step (and the fill), ascending
    position - the hot pool's own rule (oracle.pool);
  * Score: the lowest score first, where a position's score at a step is
    the largest of its index scores over the step's ways (a way's scores
    past its visible length are -inf); equal scores: lower position first;
  * Random: a 64-bit key per (request, step, position), the smallest first
    (equal keys: lower position first).  The key is output number
    (request << 48 | step << 32 | position) + 1 of the SplitMix64 generator
    (Steele, Lea and Flood, "Fast splittable pseudorandom number
    generators", OOPSLA 2014) seeded with `seed`: mix(seed + n * gamma);
  * LIM (threshold + chunk scan) is not replayed: the pages name it without
    its threshold rule.
"""
from collections import OrderedDict

import numpy as np

from .pool import CapacityError
from .topk import topk_positions

GAMMA = 0x9E3779B97F4A7C15
MASK = (1 << 64) - 1

POLICIES = ("lru", "random", "score")


def splitmix64_mix(z: int) -> int:
    """SplitMix64's output function (the finaliser applied to the state)."""
    z &= MASK
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK
    return z ^ (z >> 31)


def splitmix64_output(seed: int, n: int) -> int:
    """Output number n (1-based) of SplitMix64 seeded with `seed`: the state
    after n increments of gamma, finalised."""
    return splitmix64_mix((seed + n * GAMMA) & MASK)


def random_key(seed: int, request: int, step: int, pos: int) -> int:
    counter = (request << 48) | (step << 32) | pos
    return splitmix64_output(seed, counter + 1)


def replay(scores, sel_pos, n_sel, pool_slots, policy, seed=0, request=0):
    """Replay one request's decode steps through a pool of C slots.

    scores: float [T][m][L] index scores of every step and way (-inf past a
    way's visible length); sel_pos: int [T][m][k] selections in rank order;
    n_sel: int [T][m].  Returns (n_miss, n_evict), int arrays of length T.
    """
    if policy not in POLICIES:
        raise ValueError(policy)
    scores = np.asarray(scores, np.float64)
    T, m, L = scores.shape
    C = int(pool_slots)

    # First fill: top-C of way 0 at step 0, into the empty pool; recency in
    # ascending position.
    n_vis0 = int(np.sum(np.isfinite(scores[0, 0])))
    fill = sorted(int(p) for p in topk_positions(scores[0, 0], n_vis0, min(C, n_vis0)))
    resident = OrderedDict((p, None) for p in fill)   # front = least recent
    free = C - len(fill)

    n_miss = np.zeros(T, np.int64)
    n_evict = np.zeros(T, np.int64)
    for t in range(T):
        union = sorted({int(p) for j in range(m)
                        for p in np.asarray(sel_pos[t][j])[:int(n_sel[t][j])]})
        if len(union) > C:
            raise CapacityError(f"union of {len(union)} exceeds {C} slots")
        in_union = set(union)
        misses = [p for p in union if p not in resident]
        from_free = min(free, len(misses))
        free -= from_free
        need = len(misses) - from_free
        cand = [p for p in resident if p not in in_union]   # least recent first
        if policy == "lru":
            victims = cand[:need]
        elif policy == "score":
            best = scores[t].max(axis=0)
            victims = sorted(cand, key=lambda p: (best[p], p))[:need]
        else:
            victims = sorted(cand, key=lambda p: (random_key(seed, request, t, p), p))[:need]
        assert len(victims) == need
        for p in victims:
            del resident[p]
        for p in union:                          # ascending position
            if p in resident:
                resident.move_to_end(p)
            else:
                resident[p] = None
        assert len(resident) + free == C
        n_miss[t] = len(misses)
        n_evict[t] = need
    return n_miss, n_evict
