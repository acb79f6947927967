"""A whole decode sequence of one request (one layer): the first fill of the
hot pool, then T steady-state steps, each running

    index scores -> top-k + slot lookup -> pool update (union, victims,
    pairing, cache_slots rewrite, host -> pool copy) -> attention

in that order, as the pages lay out one offloaded decode layer
(FlashOffloading analysis, sections "five steps and the MTP union" and
"LIM", Fig. 5).  The attention reads every selected row from the oracle's
own copy of the pool, and every step asserts that each resident slot holds
exactly the host row of its position, so the result equals attention over
the host rows, as the pages require of offload.

Requests are independent (each has its own index cache, pool, reverse index,
LRU order and host rows), so the oracle runs per request.
"""
import numpy as np

from .attention import attend
from .indexer import index_scores
from .pool import HotPool
from .topk import topk_lookup, topk_positions


def run_request(keys, q_steps, w, n_vis, qa_fn, host, *, steps, topk,
                pool_slots, scale, v_dim=512, keep_scores=False,
                check_pool=True, n_vis_fn=None):
    """Generator over the fill and the steps of one request.

    keys:    uint8 [L][d_I]            fp8 index keys
    q_steps: uint8 [T][m][H_I][d_I]    fp8 index queries per step
    w:       float [m][H_I]            head weights
    n_vis:   int [m]
    qa_fn:   t -> uint16 [m][H][D]     absorbed queries of step t (bf16 bits)
    host:    uint16 [L][D]             host latents (bf16 bits)
    n_vis_fn: t -> int [m], the visible lengths of step t when the context
             grows (n_vis then serves the first fill only).  Growth changes
             which positions can be selected, nothing else: the method's
             results do not depend on where a latent is held (host store,
             pool or a tail block), so the oracle reads every row from host.

    Yields first a dict for the fill, then one dict per step t.
    """
    L, D = host.shape
    pool = HotPool(L, pool_slots)
    rows = np.zeros((pool_slots, D), np.uint16)

    # First fill: the top-min(C, n_vis) positions of token 0 at step 0 go
    # into the empty pool.
    s0 = index_scores(q_steps[0], w, keys, n_vis)
    fill_pos = topk_positions(s0[0], n_vis[0], pool_slots)
    fill = pool.update(fill_pos[None, :], np.array([fill_pos.size]))
    rows[fill["miss_slot"]] = host[fill["miss_pos"]]
    yield dict(kind="fill", fill_pos=fill_pos, **fill)

    for t in range(steps):
        nv = n_vis if n_vis_fn is None else np.asarray(n_vis_fn(t), np.int64)
        s = index_scores(q_steps[t], w, keys, nv)
        sel_pos, sel_slot, n_sel = topk_lookup(s, nv, topk, pool.cache_slots)
        resident_before = pool.resident()
        upd = pool.update(sel_pos, n_sel)
        rows[upd["miss_slot"]] = host[upd["miss_pos"]]
        if check_pool:
            pool.check_invariants()
            res = np.nonzero(pool.cache_slots >= 0)[0]
            assert np.array_equal(rows[pool.cache_slots[res]], host[res])
            union = set()
            for j in range(len(n_sel)):
                union |= set(sel_pos[j, :n_sel[j]].tolist())
            assert union <= pool.resident()
            assert upd["n_miss"] == len(union - resident_before)
        qa = qa_fn(t)
        m = len(n_sel)
        out = np.zeros((m, qa.shape[1], v_dim))
        lse = np.zeros((m, qa.shape[1]))
        for j in range(m):
            n = int(n_sel[j])
            X = rows[upd["sel_slot_post"][j, :n]]
            out[j], lse[j] = attend(qa[j], X, scale, v_dim)
        rec = dict(kind="step", t=t, sel_pos=sel_pos, sel_slot=sel_slot,
                   n_sel=n_sel, out=out, lse=lse, **upd)
        if keep_scores:
            rec["scores"] = s
        yield rec


def run_workload_request(wl, layer: int, b: int, steps=None, host=None,
                         grow_from=None, **kw):
    """run_request on the seeded synthetic inputs of workload wl (host: the
    request's latents [L][576] in place of the generated ones, e.g. the
    dequantized fp8 entries of a host store that holds entries).  grow_from
    = L0: the context starts at L0 positions (the fill sees the last m of
    them as the query tokens) and every step appends its m tokens, so step t
    token j sees n_vis = L0 + t*m + 1 + j."""
    from synth import gen
    steps = wl.steps if steps is None else steps
    keys = gen.index_keys(wl, layer, b)
    q = np.stack([gen.encode_e4m3_int(gen.index_query_ints(wl, layer, b, j))
                  for j in range(wl.mtp)], axis=1)          # [T][m][H_I][d]
    w = np.stack([gen.head_weights(wl, layer, b, j) for j in range(wl.mtp)])
    n_vis = np.array([wl.n_vis(j) for j in range(wl.mtp)], np.int64)
    if grow_from is not None:
        m = wl.mtp
        n_vis = np.array([grow_from - m + 1 + j for j in range(m)], np.int64)
        kw["n_vis_fn"] = lambda t: [grow_from + t * m + 1 + j for j in range(m)]
    host = gen.latents(wl, layer, b) if host is None else np.asarray(host)

    def qa_fn(t):
        return gen.abs_query(wl, layer, t)[b]
    return run_request(keys, q, w, n_vis, qa_fn, host, steps=steps,
                       topk=wl.topk, pool_slots=wl.pool_slots,
                       scale=wl.softmax_scale, v_dim=wl.v_dim, **kw)
