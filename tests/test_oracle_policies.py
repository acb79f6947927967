"""Pins of the eviction-policy replay oracle (oracle.policies)."""
import numpy as np
import pytest

from oracle.policies import POLICIES, random_key, replay, splitmix64_output
from oracle.pool import CapacityError, HotPool
from oracle.topk import topk_lookup, topk_positions


def test_splitmix64_reference_outputs():
    # The reference generator seeded with 0 starts 0xe220a8397b1dcdaf,
    # 0x6e789e6aa1b965f4, 0x06c45d188009454f (splitmix64.c, Vigna).
    assert splitmix64_output(0, 1) == 0xE220A8397B1DCDAF
    assert splitmix64_output(0, 2) == 0x6E789E6AA1B965F4
    assert splitmix64_output(0, 3) == 0x06C45D188009454F


def _sel(scores, k):
    """Rank-order top-k of every step and way (what the decode selects)."""
    T, m, L = scores.shape
    sel = np.full((T, m, k), -1, np.int64)
    n = np.zeros((T, m), np.int64)
    for t in range(T):
        for j in range(m):
            nv = int(np.sum(np.isfinite(scores[t, j])))
            p = topk_positions(scores[t, j], nv, k)
            sel[t, j, :p.size] = p
            n[t, j] = p.size
    return sel, n


def test_worked_example_lru_and_score_differ():
    # L = 10, C = 4, one way, k = 2.  Step 0 fills {0,1,2,3} and selects {0,1}.
    # Step 1 selects {8,9}: Score evicts the two lowest step-1 scores outside
    # the union, 0 (1) and 2 (3); LRU evicts the least recent, 2 and 3 (0 and 1
    # were used at step 0).  Step 2 selects {0,2}: under Score both miss and
    # the victims are 1 and 3 (score 0 each, lower position first); under LRU
    # only 2 misses and 1 is the least recent outside the union.
    s = np.array([
        [[9, 8, 7, 6, 1, 1, 1, 1, 1, 1]],
        [[1, 5, 3, 4, 2, 2, 2, 2, 9, 8]],
        [[9, 0, 8, 0, 0, 0, 0, 0, 1, 2]],
    ], np.float64)
    sel, n = _sel(s, 2)
    assert [sorted(sel[t, 0]) for t in range(3)] == [[0, 1], [8, 9], [0, 2]]
    miss, ev = replay(s, sel, n, 4, "score")
    assert miss.tolist() == [0, 2, 2] and ev.tolist() == [0, 2, 2]
    miss, ev = replay(s, sel, n, 4, "lru")
    assert miss.tolist() == [0, 2, 1] and ev.tolist() == [0, 2, 1]


def _random_scores(rng, T, m, L, drift=0.9):
    """Integer scores with step-to-step correlation and ties."""
    base = rng.integers(0, 200, (m, L)).astype(np.float64)
    out = np.empty((T, m, L))
    for t in range(T):
        base = np.rint(drift * base + (1 - drift) * rng.integers(0, 200, (m, L)))
        out[t] = base
    return out


@pytest.mark.parametrize("m,L,k,C", [(1, 500, 40, 120), (2, 700, 50, 160), (3, 300, 20, 64)])
def test_lru_replay_equals_the_hot_pool(m, L, k, C):
    # The LRU replay is the pool of the decode: same fill, same misses every
    # step as oracle.pool.HotPool driven by the same selections.
    rng = np.random.default_rng(L + m)
    T = 12
    s = _random_scores(rng, T, m, L)
    sel, n = _sel(s, k)
    miss, ev = replay(s, sel, n, C, "lru")
    pool = HotPool(L, C)
    fill_sel, _, fill_n = topk_lookup(s[0, :1], [L], C, pool.cache_slots)
    pool.update(fill_sel, fill_n)
    for t in range(T):
        r = pool.update(sel[t], n[t])
        assert r["n_miss"] == miss[t] and r["n_evict"] == ev[t], t


@pytest.mark.parametrize("policy", POLICIES)
def test_no_evictions_when_everything_fits(policy):
    # C >= L: nothing is ever evicted; each step misses exactly the positions
    # never seen before (not in the fill nor in an earlier union).
    rng = np.random.default_rng(5)
    T, m, L, k = 10, 2, 300, 30
    s = _random_scores(rng, T, m, L, drift=0.5)
    s[:, 1, L - 7:] = -np.inf                       # way 1 sees less
    sel, n = _sel(s, k)
    miss, ev = replay(s, sel, n, L, policy, seed=3)
    seen = set(int(p) for p in np.nonzero(np.isfinite(s[0, 0]))[0])   # the fill: all of way 0
    for t in range(T):
        u = {int(p) for j in range(m) for p in sel[t, j, :n[t, j]]}
        assert miss[t] == len(u - seen) and ev[t] == 0
        seen |= u


@pytest.mark.parametrize("policy", POLICIES)
def test_misses_are_the_union_minus_the_residents(policy):
    # Every policy: misses counted against the pool before the step, one
    # victim per miss beyond the free slots, and a union larger than C is a
    # capacity error.
    rng = np.random.default_rng(11)
    s = _random_scores(rng, 6, 2, 400)
    sel, n = _sel(s, 64)
    miss, ev = replay(s, sel, n, 128, policy, seed=1)
    assert np.all(ev <= miss) and np.all(miss <= 128)
    with pytest.raises(CapacityError):
        replay(s, sel, n, 100, policy)              # two ways of 64 can need 128


def test_random_victims_are_uniform():
    # One victim drawn from the same 8 candidates at each of 4000 steps: each
    # is drawn about equally often (chi-square with 7 degrees of freedom,
    # far below the 0.1 % critical value 24.3).
    seed, T = 12345, 4000
    counts = np.zeros(8, np.int64)
    for t in range(T):
        counts[min((random_key(seed, 0, t, p), p) for p in range(8))[1]] += 1
    exp = T / 8
    assert float(np.sum((counts - exp) ** 2 / exp)) < 24.3, counts


def test_random_replay_evicts_the_smallest_key():
    # A pool of 8 holding {0..7}.  Step 1 selects 8: the victim v1 is the
    # resident with the smallest key at step 1.  Step 2 selects v1 again: it
    # misses, and the victim v2 is the smallest key among the other
    # residents.  Step 3 selects a resident other than v2 (no miss), step 4
    # selects v2 (a miss).
    seed, req = 777, 2
    v1 = min((random_key(seed, req, 1, p), p) for p in range(8))[1]
    res = (set(range(8)) - {v1}) | {8}
    v2 = min((random_key(seed, req, 2, p), p) for p in res)[1]
    keep = min(res - {v2})
    picks = [0, 8, v1, keep, v2]
    s = np.zeros((5, 1, 10))
    s[0, 0, :8] = 10                 # fill = top-8 of step 0 = {0..7}
    for t in range(1, 5):
        s[t, 0, picks[t]] = 20
    sel, n = _sel(s, 1)
    assert [int(sel[t, 0, 0]) for t in range(5)] == picks
    miss, ev = replay(s, sel, n, 8, "random", seed=seed, request=req)
    assert miss.tolist() == [0, 1, 1, 0, 1]


def test_random_depends_on_seed_and_request():
    assert random_key(1, 0, 0, 5) != random_key(2, 0, 0, 5)
    assert random_key(1, 0, 0, 5) != random_key(1, 1, 0, 5)
    assert random_key(1, 0, 0, 5) != random_key(1, 0, 1, 5)
