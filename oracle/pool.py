"""Hot pool of C latent slots with an LRU recency order and the cache_slots
reverse index.

What the pages fix:
  * cache_slots holds, per request and layer, one int32 per position: the
    slot the position occupies, or -1 when it is not resident; a lookup is
    O(1) (FlashOffloading analysis, section "cache_slots: O(|C|) -> O(1)").
  * One steady-state step: look every way's top-k up in cache_slots; take
    the union of the misses over the MTP ways (this is the step's real
    transfer volume); pick as many victims as misses from the pool minus the
    union of the ways' top-k; pair each miss with one victim slot and
    rewrite cache_slots; copy the misses from host into their slots
    (same page, section "five steps and the MTP union").  Loads and evictions
    pair one to one, so the pool size never changes.
  * The first decode step fills the pool with |C_b| tokens from host memory
    ("first fill"), then every step swaps (same page, decode section intro).
  * ESS keeps the hot subset with an LRU policy (ESS concept page, "core
    mechanism" table).

Readings where the pages are silent:
  * recency = the last step in which a position was in the union; within
    one step positions become most-recently-used in ascending position order;
  * victims = free slots in ascending slot order first, then resident
    positions outside the union from the least-recently-used end;
  * pairing = misses in ascending position order with victims in that order;
  * the fill = the union of the fill selection placed into an empty pool, so
    slot i receives the i-th smallest filled position;
  * a miss's designated writer is the row of the smallest token j that
    selected it.
"""
from collections import OrderedDict

import numpy as np


class CapacityError(RuntimeError):
    pass


class HotPool:
    """Residency state of one request (one layer)."""

    def __init__(self, ctx_len: int, slots: int):
        self.L = int(ctx_len)
        self.C = int(slots)
        self.cache_slots = np.full(self.L, -1, np.int32)
        self.slot_pos = np.full(self.C, -1, np.int32)
        self.lru = OrderedDict()          # position -> slot; front = LRU
        self.free = list(range(self.C))   # ascending free slots

    @classmethod
    def from_state(cls, ctx_len, slots, cache_slots, lru_front_to_back):
        """Build a pool from an explicit cache_slots table and LRU order."""
        p = cls(ctx_len, slots)
        cs = np.asarray(cache_slots, np.int32)
        resident = [int(x) for x in np.nonzero(cs >= 0)[0]]
        if sorted(resident) != sorted(int(x) for x in lru_front_to_back):
            raise ValueError("LRU order must list exactly the resident positions")
        p.cache_slots[:] = cs
        for pos in lru_front_to_back:
            s = int(cs[pos])
            p.lru[int(pos)] = s
            p.slot_pos[s] = pos
        p.free = [s for s in range(p.C) if p.slot_pos[s] < 0]
        return p

    def resident(self):
        return set(self.lru.keys())

    def update(self, sel_pos, n_sel):
        """One step of the pool for the m ways' selections.

        sel_pos: int [m][k] positions in rank order; n_sel: int [m].
        Returns a dict with miss_pos, miss_slot (ascending miss positions and
        their paired slots), n_miss, n_evict, evicted (positions), row_dst
        int32 [m][k] and sel_slot_post int32 [m][k].
        """
        m = len(n_sel)
        k = np.asarray(sel_pos).shape[1]
        ways = [[int(x) for x in np.asarray(sel_pos)[j, :int(n_sel[j])]]
                for j in range(m)]
        union = sorted(set().union(*[set(w) for w in ways]))
        if len(union) > self.C:
            raise CapacityError(f"union of {len(union)} exceeds {self.C} slots")
        in_union = set(union)
        misses = [p for p in union if p not in self.lru]

        victims = []
        while len(victims) < len(misses) and self.free:
            victims.append(self.free.pop(0))
        n_free_used = len(victims)
        evicted = []
        if len(victims) < len(misses):
            for p in list(self.lru.keys()):        # least recent first
                if len(victims) == len(misses):
                    break
                if p in in_union:
                    continue
                s = self.lru.pop(p)
                self.cache_slots[p] = -1
                self.slot_pos[s] = -1
                victims.append(s)
                evicted.append(p)
        assert len(victims) == len(misses)

        for p, s in zip(misses, victims):
            self.cache_slots[p] = s
            self.slot_pos[s] = p

        for p in union:                             # ascending position
            if p in self.lru:
                self.lru.move_to_end(p)
            else:
                self.lru[p] = int(self.cache_slots[p])

        row_dst = np.full((m, k), -1, np.int32)
        writer_done = set()
        miss_set = set(misses)
        for j in range(m):
            for i, p in enumerate(ways[j]):
                if p in miss_set and p not in writer_done:
                    row_dst[j, i] = self.cache_slots[p]
                    writer_done.add(p)
        post = np.full((m, k), -1, np.int32)
        for j in range(m):
            if ways[j]:
                post[j, :len(ways[j])] = self.cache_slots[np.array(ways[j])]
        return dict(miss_pos=np.array(misses, np.int64),
                    miss_slot=np.array(victims, np.int64),
                    n_miss=len(misses), n_evict=len(evicted),
                    n_free_used=n_free_used, evicted=evicted,
                    row_dst=row_dst, sel_slot_post=post)

    def check_invariants(self):
        """Reverse index and slot table are inverse bijections on residents."""
        res = np.nonzero(self.cache_slots >= 0)[0]
        assert len(res) == len(self.lru) <= self.C
        assert np.all(self.slot_pos[self.cache_slots[res]] == res)
        used = np.nonzero(self.slot_pos >= 0)[0]
        assert len(used) == len(res)
        assert np.all(self.cache_slots[self.slot_pos[used]] == used)
        assert set(self.free) == set(range(self.C)) - set(used.tolist())
