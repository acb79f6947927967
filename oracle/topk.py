"""Top-k selection with the residency lookup read off the winners.

The pages select the top k of the indexer scores, pack each candidate's index
and cache_slots value with its score so that the winners directly give the
slot list, and print a 20-candidate example whose top 3 come out as
[8, 4, 17] with slots [-1, 7, -1] (FlashOffloading analysis, section "LIM:
packing the index into the score").  That example lists the winners in rank
order, not position order; the reading taken is rank order (descending
score).  The pages leave ties open; the reading taken is that on equal scores
the lower position wins.

The oracle is the plain definition: a full sort on (score descending,
position ascending), then a lookup of cache_slots at each winner.
"""
import numpy as np


def topk_positions(scores_row, n_vis: int, k: int) -> np.ndarray:
    """Positions of the min(k, n_vis) best candidates, in rank order."""
    n = int(n_vis)
    s = np.asarray(scores_row[:n], dtype=np.float64)
    # lexsort: last key is primary -> score descending, then position.
    order = np.lexsort((np.arange(n), -s))
    return order[:min(int(k), n)].astype(np.int64)


def topk_lookup(scores, n_vis, k: int, cache_slots):
    """Top-k of every query token of one request plus the slot lookup.

    scores: [m][L]; n_vis: [m]; cache_slots: int [L] (state before the step)
    returns (sel_pos int32 [m][k], sel_slot int32 [m][k], n_sel int32 [m]),
    rows at or beyond n_sel padded with -1.
    """
    m = len(n_vis)
    sel_pos = np.full((m, k), -1, np.int32)
    sel_slot = np.full((m, k), -1, np.int32)
    n_sel = np.zeros(m, np.int32)
    for j in range(m):
        p = topk_positions(scores[j], n_vis[j], k)
        n_sel[j] = p.size
        sel_pos[j, :p.size] = p
        sel_slot[j, :p.size] = np.asarray(cache_slots)[p]
    return sel_pos, sel_slot, n_sel
