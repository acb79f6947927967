"""Pins for the oracle's hot pool: the pages' Fig. 4 step, an independent
stamp-based LRU written another way, the invariants the pages state (size
constant after the fill, victims outside the union, misses = union minus
the previous pool) and the capacity limit."""
import numpy as np
import pytest

from oracle.pool import CapacityError, HotPool
from tests.golden.load import load


def test_fig4_step():
    g = load("fig4_example.txt")
    cs = np.array(g["cache_slots"], np.int32)
    resident = [int(p) for p in np.nonzero(cs >= 0)[0]]
    # LRU order with tokens 18 and 19 least recent (the figure evicts them).
    lru = [18, 19] + [p for p in resident if p not in (18, 19)]
    pool = HotPool.from_state(g["ctx_len"], g["pool_slots"], cs, lru)
    sel = np.array([g["selected"]])
    r = pool.update(sel, [3])
    assert r["miss_pos"].tolist() == g["expect_miss_pos"]
    assert r["miss_slot"].tolist() == g["expect_miss_slot"]
    assert r["n_miss"] == g["expect_n_miss"] and r["n_evict"] == 2
    blocks = [p // g["dram_block_tokens"] + 1 for p in r["miss_pos"]]
    assert blocks == g["expect_dram_block"]
    hp, hs = (int(x) for x in g["expect_hit"].split(":"))
    assert pool.cache_slots[hp] == hs
    assert pool.cache_slots[18] == -1 and pool.cache_slots[19] == -1
    assert pool.cache_slots[8] == 3 and pool.cache_slots[17] == 5
    assert len(pool.resident()) == g["pool_slots"]
    # Only the miss row writes its slot; the hit row does not.
    assert r["row_dst"][0].tolist() == [3, -1, 5]
    assert r["sel_slot_post"][0].tolist() == [3, 7, 5]
    pool.check_invariants()


class StampPool:
    """LRU written another way: recency is the pair (last step used,
    position) and victims are found by sorting, not by list order."""

    def __init__(self, L, C):
        self.C = C
        self.slot_of = {}
        self.last = {}
        self.used_slots = set()
        self.step = 0

    def update(self, ways):
        U = set()
        for w in ways:
            U |= set(w)
        misses = sorted(p for p in U if p not in self.slot_of)
        free = sorted(set(range(self.C)) - self.used_slots)
        victims = free[:len(misses)]
        need = len(misses) - len(victims)
        cand = sorted((self.last[p], p) for p in self.slot_of if p not in U)
        evicted = [p for _, p in cand[:need]]
        for p in evicted:
            victims.append(self.slot_of.pop(p))
            del self.last[p]
        for p, s in zip(misses, victims):
            self.slot_of[p] = s
            self.used_slots.add(s)
        for p in U:
            self.last[p] = self.step
        self.step += 1
        return misses, victims, evicted


def _random_ways(rng, L, m, k, prev):
    ways = []
    for j in range(m):
        keep = [p for p in prev[j] if rng.random() < 0.8] if prev else []
        pool = [p for p in rng.permutation(L).tolist() if p not in set(keep)]
        w = (keep + pool)[:k]
        rng.shuffle(w)
        ways.append(w)
    return ways


@pytest.mark.parametrize("seed", range(6))
def test_orderdict_lru_matches_stamp_lru(seed):
    rng = np.random.default_rng(seed)
    L, m, k = int(rng.integers(30, 120)), int(rng.integers(1, 3)), int(rng.integers(3, 12))
    C = int(rng.integers(m * k, m * k + 25))
    a, b = HotPool(L, C), StampPool(L, C)
    prev = None
    for t in range(25):
        ways = _random_ways(rng, L, m, k, prev)
        prev = ways
        arr = np.array(ways)
        r = a.update(arr, [k] * m)
        misses, victims, evicted = b.update(ways)
        assert r["miss_pos"].tolist() == misses
        assert r["miss_slot"].tolist() == victims
        assert sorted(r["evicted"]) == sorted(evicted)
        a.check_invariants()
        assert {p: s for p, s in a.lru.items()} == b.slot_of


def test_pool_invariants_over_a_sequence():
    rng = np.random.default_rng(21)
    L, m, k, C = 500, 2, 40, 160
    pool = HotPool(L, C)
    fill = rng.permutation(L)[:C]
    r = pool.update(fill[None, :], [C])
    # The fill: slot i receives the i-th smallest filled position.
    assert r["miss_pos"].tolist() == sorted(fill.tolist())
    assert r["miss_slot"].tolist() == list(range(C))
    assert r["n_evict"] == 0 and len(pool.resident()) == C
    prev = None
    for t in range(40):
        ways = _random_ways(rng, L, m, k, prev)
        prev = ways
        before = pool.resident()
        union = set(ways[0]) | set(ways[1])
        r = pool.update(np.array(ways), [k, k])
        assert len(pool.resident()) == C                  # size constant
        assert union <= pool.resident()                   # union resident
        assert r["n_miss"] == len(union - before)         # misses
        assert set(r["evicted"]).isdisjoint(union)        # victims outside
        assert r["n_evict"] == r["n_miss"]                # pool was full
        # Exactly one designated writer per miss, at its smallest way.
        wr = [(j, i) for j in range(m) for i in range(k) if r["row_dst"][j, i] >= 0]
        assert len(wr) == r["n_miss"]
        for j, i in wr:
            p = ways[j][i]
            assert p in r["miss_pos"].tolist()
            assert all(p not in ways[jj] for jj in range(j))
        pool.check_invariants()


def test_free_slots_are_used_before_evictions():
    pool = HotPool(50, 10)
    r = pool.update(np.array([[5, 3, 9]]), [3])
    assert r["miss_slot"].tolist() == [0, 1, 2] and r["n_evict"] == 0
    r = pool.update(np.array([[1, 2, 3, 4, 6, 7, 8, 10]]), [8])
    # 7 misses, 7 free slots remain: no eviction.
    assert r["n_miss"] == 7 and r["n_evict"] == 0
    assert r["miss_slot"].tolist() == list(range(3, 10))
    r = pool.update(np.array([[11, 3]]), [2])
    # Pool full: the least recent non-selected position (5, used in step 0
    # and never again; 9 too, 5 < 9) is evicted.
    assert r["n_evict"] == 1 and r["evicted"] == [5]


def test_capacity_error():
    pool = HotPool(40, 5)
    with pytest.raises(CapacityError):
        pool.update(np.array([[1, 2, 3], [4, 5, 6]]), [3, 3])


def test_all_resident_pool_has_no_steady_misses():
    L = 64
    pool = HotPool(L, 80)
    pool.update(np.arange(L)[None, :], [L])
    rng = np.random.default_rng(2)
    for t in range(10):
        r = pool.update(rng.permutation(L)[None, :16], [16])
        assert r["n_miss"] == 0 and r["n_evict"] == 0
