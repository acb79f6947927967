"""Per-call GPU parity against the CPU oracle: indexer scores and top-k
bit-exact, pool updates bit-exact over step sequences, attention within the
stated tolerance with miss write-back and placement invariance."""
import zlib

import numpy as np
import pytest
import torch

from decode_lightning_indexer_amd import ess
from decode_lightning_indexer_amd.session import HostStore
from oracle.attention import attend
from oracle.indexer import index_scores
from oracle.pool import HotPool
from oracle.topk import topk_lookup
from synth import gen
from tests.gpu_util import assert_attn_close, dims, h, lse_close, sync, t

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------- indexer --

@pytest.mark.parametrize("B,m,L,HI,dI,ragged", [
    (1, 1, 4096, 16, 64, False),
    (2, 1, 5000, 64, 128, False),
    (2, 2, 3001, 64, 128, False),
    (3, 1, 17, 16, 64, True),
    (2, 1, 1500, 32, 128, True),
    (1, 4, 777, 32, 64, True),
])
def test_index_scores_bit_exact(B, m, L, HI, dI, ragged):
    rng = np.random.default_rng(L + B + m)
    qi = rng.integers(-7, 8, (B, m, HI, dI))
    ki = rng.integers(-7, 8, (B, L, dI))
    w = rng.integers(1, 5, (B, m, HI)).astype(np.float32)
    if ragged:
        n_vis = rng.integers(1, L + 1, (B, m)).astype(np.int32)
    else:
        n_vis = np.array([[L - m + 1 + j for j in range(m)]] * B, np.int32)
    q8, k8 = gen.encode_e4m3_int(qi), gen.encode_e4m3_int(ki)
    d = dims(batch=B, mtp=m, ctx_len=L, idx_heads=HI, idx_dim=dI)
    scores = torch.empty((B, m, L), dtype=torch.float32, device="cuda")
    ess.ess_index_scores(d, t(q8), t(w), t(k8), t(n_vis), scores)
    sync()
    got = h(scores)
    for b in range(B):
        ref = index_scores(q8[b], w[b], k8[b], n_vis[b])
        assert np.array_equal(got[b].astype(np.float64), ref), b


def test_index_scores_long_context_offsets():
    # A context past 2^25 positions of 128-byte keys: byte offsets into the
    # index cache pass 2^32.  Every key is zero except the last 12288 rows
    # (seeded), so a wrapped offset would read a zero row; the last 8192
    # scores, on both sides of position 2^25, must equal the oracle's.
    L, HI, dI, tail = (1 << 25) + 4096, 16, 128, 12288
    print(f"\n[indexer] L={L} d_I={dI}", flush=True)
    rng = np.random.default_rng(1 << 25)
    qi = rng.integers(-7, 8, (1, 1, HI, dI))
    ki = rng.integers(-7, 8, (tail, dI))
    ki[rng.random(tail) < 0.05] = 0        # a few zero rows: scores of 0
    w = rng.integers(1, 5, (1, 1, HI)).astype(np.float32)
    q8, k8 = gen.encode_e4m3_int(qi), gen.encode_e4m3_int(ki)
    keys = torch.zeros((1, L, dI), dtype=torch.uint8, device="cuda")
    keys[0, L - tail:] = torch.from_numpy(k8).to("cuda")
    n_vis = np.array([[L]], np.int32)
    d = dims(batch=1, mtp=1, ctx_len=L, idx_heads=HI, idx_dim=dI)
    scores = torch.empty((1, 1, L), dtype=torch.float32, device="cuda")
    ess.ess_index_scores(d, t(q8), t(w), keys, t(n_vis), scores)
    sync()
    got = h(scores[0, 0, L - 8192:])
    ref = index_scores(q8[0], w[0], k8[tail - 8192:], [8192])[0]
    assert np.array_equal(got.astype(np.float64), ref)
    assert float(scores[0, 0, :L - tail].abs().max()) == 0.0
    del keys, scores


# --------------------------------------------------------------- top-k --

def _scores(kind, rng, shape):
    if kind == "int_ties":
        return rng.integers(0, 40, shape).astype(np.float32)
    if kind == "indexer_like":
        return np.rint(rng.normal(13000, 2500, shape)).clip(0).astype(np.float32)
    if kind == "float":
        return rng.standard_normal(shape).astype(np.float32)
    if kind == "wide":
        return (rng.lognormal(0, 8, shape) * rng.choice([-1, 1], shape)).astype(np.float32)
    if kind == "equal":
        return np.full(shape, 3.5, np.float32)
    if kind == "zeros":
        a = rng.choice(np.array([0.0, -0.0, 1.0, -1.0], np.float32), shape)
        return a.astype(np.float32)
    raise ValueError(kind)


@pytest.mark.parametrize("kind,B,m,n_tok,L,k,ragged", [
    ("int_ties", 2, 1, 1, 5000, 256, False),
    ("indexer_like", 4, 1, 1, 32768, 2048, False),
    ("indexer_like", 4, 1, 1, 32768, 2048, True),   # row in registers, ragged counts
    ("indexer_like", 2, 2, 2, 40000, 2048, True),
    ("float", 2, 1, 1, 3000, 100, True),
    ("wide", 2, 1, 1, 20000, 1000, False),
    ("equal", 1, 1, 1, 10000, 300, False),
    ("equal", 1, 1, 1, 3000, 2500, False),
    ("zeros", 2, 1, 1, 7000, 512, False),
    ("int_ties", 2, 1, 1, 100, 2048, True),       # k >= n_vis
    ("indexer_like", 1, 2, 1, 30000, 16384, False),  # fill-size k, token 0 only
    ("int_ties", 3, 1, 1, 1, 1, False),
    ("float", 1, 3, 3, 2049, 7, True),
    # Rows longer than 32768 keys (k <= 4096) are split over workgroups of
    # 16384 keys that select together.
    ("int_ties", 2, 1, 1, 70000, 1000, True),
    ("equal", 1, 1, 1, 100000, 2048, False),      # one run of equal keys
    ("zeros", 1, 1, 1, 50000, 513, False),        # +-0, k not a multiple of 4
    ("wide", 1, 1, 1, 1 << 20, 2048, False),      # two levels
    ("indexer_like", 2, 2, 2, 131072, 2048, True),
    ("indexer_like", 1, 1, 1, 1 << 20, 4096, False),
    ("float", 1, 1, 1, 300000, 7, True),
    ("float", 1, 1, 1, 40000, 5000, False),       # k > 4096: one workgroup
    ("float", 2, 3, 1, 40000, 100, True),         # n_tok < m on long rows
    # 10 rows x 14 spans: more workgroups than the split selection takes in
    # one launch, so these rows select in levels.
    ("indexer_like", 5, 2, 2, 220000, 1024, True),
])
def test_topk_bit_exact(kind, B, m, n_tok, L, k, ragged):
    rng = np.random.default_rng(zlib.crc32(f"{kind}-{L}-{k}".encode()))
    s = _scores(kind, rng, (B, m, L))
    if ragged:
        n_vis = rng.integers(1, L + 1, (B, m)).astype(np.int32)
    else:
        n_vis = np.full((B, m), L, np.int32)
    cs = np.where(rng.random((B, L)) < 0.5, rng.integers(0, 1 << 20, (B, L)), -1).astype(np.int32)
    d = dims(batch=B, mtp=m, ctx_len=L, topk=min(k, 16384), pool_slots=16384)
    sp = torch.empty((B, n_tok, k), dtype=torch.int32, device="cuda")
    ss = torch.empty_like(sp)
    ns = torch.empty((B, n_tok), dtype=torch.int32, device="cuda")
    wsb = ess.ess_workspace_bytes(d)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    ess.ess_topk_lookup(d, k, n_tok, t(s), t(n_vis), t(cs), sp, ss, ns, ws, wsb)
    sync()
    for b in range(B):
        rp, rs, rn = topk_lookup(s[b, :n_tok].astype(np.float64), n_vis[b, :n_tok], k, cs[b])
        assert np.array_equal(h(ns)[b], rn), b
        assert np.array_equal(h(sp)[b], rp), b
        assert np.array_equal(h(ss)[b], rs), b


@pytest.mark.parametrize("L", [3000, 32768, 40000])
def test_topk_visible_counts_at_the_edges(L):
    # Rows whose visible count is 0, 1, just below, at and just above k, and
    # the whole row: a row of 32768 keys is held in registers and loaded
    # before its count arrives, 3000 keys take the bounded scalar loads, and
    # 40000 keys split over workgroups.
    k = 2048
    counts = [0, 1, k - 1, k, k + 1, L]
    B = len(counts)
    rng = np.random.default_rng(zlib.crc32(f"edges-{L}".encode()))
    s = _scores("indexer_like", rng, (B, 1, L))
    n_vis = np.array([[min(c, L)] for c in counts], np.int32)
    cs = np.where(rng.random((B, L)) < 0.5, rng.integers(0, 1 << 20, (B, L)), -1).astype(np.int32)
    d = dims(batch=B, mtp=1, ctx_len=L, topk=k, pool_slots=16384)
    sp = torch.empty((B, 1, k), dtype=torch.int32, device="cuda")
    ss = torch.empty_like(sp)
    ns = torch.empty((B, 1), dtype=torch.int32, device="cuda")
    wsb = ess.ess_workspace_bytes(d)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    ess.ess_topk_lookup(d, k, 1, t(s), t(n_vis), t(cs), sp, ss, ns, ws, wsb)
    sync()
    for b in range(B):
        rp, rs, rn = topk_lookup(s[b, :1].astype(np.float64), n_vis[b, :1], k, cs[b])
        assert np.array_equal(h(ns)[b], rn), b
        assert np.array_equal(h(sp)[b], rp), b
        assert np.array_equal(h(ss)[b], rs), b


# ---------------------------------------------------------------- pool --

def _ways(rng, L, m, k, prev, keep=0.85):
    ways = []
    for j in range(m):
        kp = [p for p in prev[j] if rng.random() < keep] if prev else []
        s = set(kp)
        fresh = [p for p in rng.permutation(L)[:2 * k + 8].tolist() if p not in s]
        w = (kp + fresh)[:k]
        rng.shuffle(w)
        ways.append(w)
    return ways


@pytest.mark.parametrize("B,m,L,C,k,steps,ragged", [
    (2, 1, 3000, 256, 64, 30, False),
    (2, 2, 5000, 512, 100, 25, True),
    (1, 1, 500, 64, 16, 60, False),        # many steps: ring compaction
    (3, 2, 4000, 300, 150, 12, False),     # union near capacity
    (1, 1, 200, 400, 50, 10, False),       # pool larger than the context
])
def test_pool_update_bit_exact(B, m, L, C, k, steps, ragged):
    rng = np.random.default_rng(B * 1000 + C)
    d = dims(batch=B, mtp=m, ctx_len=L, topk=k, pool_slots=C)
    cs = torch.empty((B, L), dtype=torch.int32, device="cuda")
    sp = torch.empty((B, C), dtype=torch.int32, device="cuda")
    lru = torch.empty(ess.ess_lru_state_bytes(d), dtype=torch.uint8, device="cuda")
    ess.ess_pool_reset(d, cs, sp, lru)
    lists = max(m * k, C)
    mp = torch.empty(B * lists, dtype=torch.int32, device="cuda")
    ms, rd, post = torch.empty_like(mp), torch.empty_like(mp), torch.empty_like(mp)
    nm = torch.empty(B, dtype=torch.int32, device="cuda")
    ne = torch.empty_like(nm)
    pools = [HotPool(L, C) for _ in range(B)]

    def run(kk, n_tok, sel, nsel):
        ess.ess_pool_update(d, kk, n_tok, t(sel), t(nsel), cs, sp, lru, mp, ms,
                            nm, ne, rd, post)
        sync()
        gm, gs = h(mp)[:B * n_tok * kk].reshape(B, -1), h(ms)[:B * n_tok * kk].reshape(B, -1)
        grd = h(rd)[:B * n_tok * kk].reshape(B, n_tok, kk)
        gpost = h(post)[:B * n_tok * kk].reshape(B, n_tok, kk)
        for b in range(B):
            r = pools[b].update(sel[b], nsel[b])
            n = int(h(nm)[b])
            assert n == r["n_miss"] and int(h(ne)[b]) == r["n_evict"], b
            assert np.array_equal(gm[b, :n], r["miss_pos"]), b
            assert np.array_equal(gs[b, :n], r["miss_slot"]), b
            assert np.array_equal(grd[b], r["row_dst"]), b
            assert np.array_equal(gpost[b], r["sel_slot_post"]), b
            assert np.array_equal(h(cs)[b], pools[b].cache_slots), b
            assert np.array_equal(h(sp)[b], pools[b].slot_pos), b

    # Fill: one way of min(C, L) positions into the empty pool.
    kf = min(C, L)
    fill = np.stack([rng.permutation(L)[:kf] for _ in range(B)])[:, None, :].astype(np.int32)
    run(kf, 1, fill, np.full((B, 1), kf, np.int32))
    prev = [None] * B
    for step in range(steps):
        sel = np.full((B, m, k), -1, np.int32)
        nsel = np.zeros((B, m), np.int32)
        for b in range(B):
            ways = _ways(rng, L, m, k, prev[b])
            prev[b] = ways
            for j in range(m):
                n = int(rng.integers(1, k + 1)) if ragged else k
                sel[b, j, :n] = ways[j][:n]
                nsel[b, j] = n
        run(k, m, sel, nsel)
    # The pool status: consistent, one update per call, and the ring
    # compacted in the long run (60 updates of 16 on a ring of 4 * 64).
    st = torch.empty((B, 4), dtype=torch.int32, device="cuda")
    ess.ess_pool_status(d, lru, st)
    sync()
    st = h(st)
    assert (st[:, 0] == 0).all() and (st[:, 2] == steps + 1).all(), st
    if (C, k, steps) == (64, 16, 60):
        assert (st[:, 1] >= 1).all(), st


def test_pool_status_flags_a_corrupted_ring():
    # A foreign write kills every recency entry (all slot stamps overwritten)
    # after the fill: the next update's victim scan runs dry.  The update
    # flags it, pairs no miss, and reports only paired misses (none), so no
    # stale copy-list entry is ever handed on.
    B, L, C, k = 1, 600, 64, 16
    d = dims(batch=B, ctx_len=L, topk=k, pool_slots=C)
    cs = torch.empty((B, L), dtype=torch.int32, device="cuda")
    sp = torch.empty((B, C), dtype=torch.int32, device="cuda")
    lru = torch.empty(ess.ess_lru_state_bytes(d), dtype=torch.uint8, device="cuda")
    ess.ess_pool_reset(d, cs, sp, lru)
    mp = torch.full((B * C,), 7, dtype=torch.int32, device="cuda")
    ms, rd, post = torch.full_like(mp, 7), torch.empty_like(mp), torch.empty_like(mp)
    nm = torch.empty(B, dtype=torch.int32, device="cuda")
    ne = torch.empty_like(nm)
    fill = np.arange(C, dtype=np.int32)[None, None, :]
    ess.ess_pool_update(d, C, 1, t(fill), t(np.array([[C]], np.int32)), cs, sp, lru,
                        mp, ms, nm, ne, rd, post)
    sync()
    st = torch.empty((B, 4), dtype=torch.int32, device="cuda")
    ess.ess_pool_status(d, lru, st)
    sync()
    assert h(st)[0].tolist() == [0, 0, 1, C]
    # Header (8 int32), then the C slot stamps: overwrite the stamps.
    lru.view(torch.int32)[8:8 + C] = -5
    sel = np.arange(C, C + k, dtype=np.int32)[None, None, :]     # k misses
    ess.ess_pool_update(d, k, 1, t(sel), t(np.array([[k]], np.int32)), cs, sp, lru,
                        mp, ms, nm, ne, rd, post)
    ess.ess_pool_status(d, lru, st)
    sync()
    assert h(st)[0, 0] == 1                 # victim scan ran dry
    assert int(h(nm)[0]) == 0 and int(h(ne)[0]) == 0
    assert (h(cs)[0, C:C + k] == -1).all()  # the misses stay unresident
    assert (h(post)[:k] == -1).all()


def test_pool_update_rejects_capacity():
    d = dims(batch=1, mtp=2, ctx_len=100, topk=64, pool_slots=100)
    z = torch.zeros(1024, dtype=torch.int32, device="cuda")
    with pytest.raises(ess.EssError) as e:
        ess.ess_pool_update(d, 64, 2, z, z, z, z, z, z, z, z, z, z, z)
    assert "capacity" in str(e.value)


# ----------------------------------------------------------- attention --

def _bf16(rng, shape, std):
    return gen.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(std))


@pytest.mark.parametrize("B,m,H,L,k,C,ragged,p_hit", [
    (1, 1, 16, 4096, 256, 1024, False, 0.8),
    (2, 1, 64, 3000, 300, 1024, True, 0.5),
    (2, 2, 128, 2000, 2048 // 4, 1200, True, 0.7),
    (1, 1, 32, 500, 45, 100, False, 0.0),     # all misses
    (1, 1, 48, 500, 33, 100, False, 1.0),     # all hits
    (1, 2, 16, 100, 200, 400, True, 0.6),     # k > L: n_sel ragged below k
    # 8 requests x 2 tokens x 2 head groups: 8 chunks of 256 of the 2048
    # rows, the chunk plan of the 128K workload.
    (8, 2, 128, 6000, 2048, 4200, True, 0.7),
    # One request: 32 chunks of 64 rows, combined by 4 waves per head (the
    # 1M workload's plan), and 16 chunks by 2 waves per head.
    (1, 1, 64, 20000, 2048, 4096, False, 0.6),
    (1, 2, 128, 9000, 1024, 2500, True, 0.5),
    # Workgroups of 32 heads (two waves per head block, column halves) and
    # of 48 heads (one wave per head block, all value columns).
    (8, 1, 32, 2500, 2048, 2100, True, 0.6),
    (4, 1, 96, 3000, 2048, 2100, True, 0.6),
])
def test_sparse_mla_parity_and_writeback(B, m, H, L, k, C, ragged, p_hit):
    _mla_case(B, m, H, L, k, C, ragged, p_hit)


@pytest.mark.parametrize("lat_std", [0.5e-4, 0.5e4, 0.5e5])
def test_sparse_mla_latent_scales(lat_std):
    # Latents far from unit scale: tiny values (whose partial outputs would
    # be fp16 subnormals unscaled) and values whose weighted means pass
    # fp16's largest finite value (65504).
    print(f"\n[mla] latent std {lat_std}", flush=True)
    _mla_case(2, 1, 64, 3000, 512, 1024, True, 0.5, lat_std=lat_std)


def _mla_case(B, m, H, L, k, C, ragged, p_hit, lat_std=0.5, q_std=0.1):
    rng = np.random.default_rng(H * 7 + k)
    host = HostStore((B, L, 576))
    host.array[:] = _bf16(rng, (B, L, 576), lat_std)
    qa = _bf16(rng, (B, m, H, 576), q_std)
    n_sel = np.zeros((B, m), np.int32)
    sel = np.full((B, m, k), -1, np.int32)
    src = np.full((B, m, k), -1, np.int32)
    dst = np.full((B, m, k), -1, np.int32)
    pool = np.zeros((B, C, 576), np.uint16)
    for b in range(B):
        slot_of = {}
        free = list(rng.permutation(C))
        for j in range(m):
            n = int(rng.integers(1, min(k, L) + 1)) if ragged else min(k, L)
            n_sel[b, j] = n
            pos = rng.permutation(L)[:n]
            sel[b, j, :n] = pos
            for i, p in enumerate(pos.tolist()):
                if p not in slot_of:
                    hit = rng.random() < p_hit
                    s = free.pop()
                    slot_of[p] = (s, hit)
                    if hit:
                        pool[b, s] = host.array[b, p]
                    else:
                        dst[b, j, i] = s       # designated writer
                s, hit = slot_of[p]
                src[b, j, i] = s if hit else -1
        # Rows at or past n_sel are never used: writer slots planted there
        # must stay untouched.
        for j in range(m):
            for i in range(n_sel[b, j], min(n_sel[b, j] + 2, k)):
                if free:
                    sel[b, j, i] = i % L
                    dst[b, j, i] = free.pop()
    d = dims(batch=B, mtp=m, ctx_len=L, mla_heads=H, topk=k, pool_slots=C)
    ws_bytes = ess.ess_workspace_bytes(d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    pool_t = t(pool)
    out = torch.empty((B, m, H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, m, H), dtype=torch.float32, device="cuda")
    ess.ess_sparse_mla_decode(d, t(qa), t(sel), t(src), t(dst), t(n_sel),
                              pool_t, host.dev, out, lse, ws, ws_bytes)
    sync()
    got, glse = h(out), h(lse)
    for b in range(B):
        for j in range(m):
            n = n_sel[b, j]
            ref, rlse = attend(qa[b, j], host.array[b, sel[b, j, :n]], 1 / 24)
            assert_attn_close(got[b, j], ref, (b, j))
            lse_close(glse[b, j], rlse, (b, j))
    # Misses landed in their slots, bit for bit; every other slot unchanged.
    gp = h(pool_t)
    for b in range(B):
        written = np.zeros(C, bool)
        for j in range(m):
            for i in np.nonzero(dst[b, j, :n_sel[b, j]] >= 0)[0]:
                assert np.array_equal(gp[b, dst[b, j, i]], host.array[b, sel[b, j, i]])
                written[dst[b, j, i]] = True
        assert np.array_equal(gp[b, ~written], pool[b, ~written]), b
    # Placement invariance: every row now read from the pool.
    src2 = src.copy()
    for b in range(B):
        slot_of = {}
        for j in range(m):
            for i in range(n_sel[b, j]):
                if dst[b, j, i] >= 0:
                    slot_of[sel[b, j, i]] = dst[b, j, i]
        for j in range(m):
            for i in range(n_sel[b, j]):
                if src2[b, j, i] < 0:
                    src2[b, j, i] = slot_of[sel[b, j, i]]
    out2 = torch.empty_like(out)
    lse2 = torch.empty_like(lse)
    ess.ess_sparse_mla_decode(d, t(qa), t(sel), t(src2), None, t(n_sel),
                              pool_t, host.dev, out2, lse2, ws, ws_bytes)
    sync()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    host.free()


def test_miss_copy():
    rng = np.random.default_rng(3)
    B, L, C, n = 2, 1000, 300, 77
    host = HostStore((B, L, 576))
    host.array[:] = _bf16(rng, (B, L, 576), 0.5)
    d = dims(batch=B, ctx_len=L, pool_slots=C)
    mp = np.stack([rng.permutation(L)[:n] for _ in range(B)]).astype(np.int32)
    ms = np.stack([rng.permutation(C)[:n] for _ in range(B)]).astype(np.int32)
    nm = np.array([n, n // 2], np.int32)
    pool = torch.zeros((B, C, 576), dtype=torch.int16, device="cuda")
    ess.ess_miss_copy(d, n, t(mp), t(ms), t(nm), host.dev, pool)
    sync()
    gp = h(pool)
    for b in range(B):
        assert np.array_equal(gp[b, ms[b, :nm[b]]], host.array[b, mp[b, :nm[b]]])
        untouched = np.setdiff1d(np.arange(C), ms[b, :nm[b]])
        assert not gp[b, untouched].any()
    host.free()


@pytest.mark.parametrize("kind", ["int_ties", "equal", "indexer_like"])
def test_topk_split_rows_at_the_edges(kind):
    # Rows of 70000 keys are split over five workgroups; visible lengths of
    # 0, 1, k - 1, k, k + 1, one span and all of them, so some rows select
    # everything, some spans see nothing, and ties cross span boundaries.
    L, k = 70000, 2048
    n_vis = np.array([[0], [1], [k - 1], [k], [k + 1], [16384], [16385], [L]], np.int32)
    B = n_vis.shape[0]
    rng = np.random.default_rng(zlib.crc32(f"split-{kind}".encode()))
    s = _scores(kind, rng, (B, 1, L))
    cs = np.where(rng.random((B, L)) < 0.5, rng.integers(0, 8192, (B, L)), -1).astype(np.int32)
    d = dims(batch=B, mtp=1, ctx_len=L, topk=k, pool_slots=8192)
    sp = torch.empty((B, 1, k), dtype=torch.int32, device="cuda")
    ss = torch.empty_like(sp)
    ns = torch.empty((B, 1), dtype=torch.int32, device="cuda")
    wsb = ess.ess_workspace_bytes(d)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    for rep in range(2):      # the workspace's counters start from what the last call left
        ess.ess_topk_lookup(d, k, 1, t(s), t(n_vis), t(cs), sp, ss, ns, ws, wsb)
        sync()
        for b in range(B):
            rp, rs, rn = topk_lookup(s[b, :1].astype(np.float64), n_vis[b, :1], k, cs[b])
            where = (kind, rep, b, int(n_vis[b, 0]))
            assert np.array_equal(h(ns)[b], rn), where
            assert np.array_equal(h(sp)[b], rp), where
            assert np.array_equal(h(ss)[b], rs), where


def test_topk_random_shapes_around_the_level_boundary():
    # Seeded shapes on both sides of the 32768-key register-resident row and
    # the 16384-key level chunk: ragged visibility (k >= n_vis inside a
    # level), k not a multiple of 4, one or several tokens, every score kind.
    rng = np.random.default_rng(20261202)
    kinds = ["int_ties", "indexer_like", "float", "wide", "zeros"]
    for case in range(14):
        kind = kinds[case % len(kinds)]
        L = int(rng.choice([16383, 16385, 32767, 32768, 32769, 49153,
                            int(rng.integers(33000, 140000))]))
        B, m = int(rng.integers(1, 3)), int(rng.integers(1, 3))
        n_tok = int(rng.integers(1, m + 1))
        k = int(rng.choice([1, 3, 257, 1024, 2047, 4096]))
        s = _scores(kind, rng, (B, m, L))
        n_vis = rng.integers(1, L + 1, (B, m)).astype(np.int32)
        cs = np.where(rng.random((B, L)) < 0.3, rng.integers(0, 16384, (B, L)), -1).astype(np.int32)
        d = dims(batch=B, mtp=m, ctx_len=L, topk=k, pool_slots=16384)
        sp = torch.empty((B, n_tok, k), dtype=torch.int32, device="cuda")
        ss = torch.empty_like(sp)
        ns = torch.empty((B, n_tok), dtype=torch.int32, device="cuda")
        wsb = ess.ess_workspace_bytes(d)
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
        ess.ess_topk_lookup(d, k, n_tok, t(s), t(n_vis), t(cs), sp, ss, ns, ws, wsb)
        sync()
        for b in range(B):
            rp, rs, rn = topk_lookup(s[b, :n_tok].astype(np.float64), n_vis[b, :n_tok], k, cs[b])
            where = (case, kind, L, B, m, n_tok, k, b)
            assert np.array_equal(h(ns)[b], rn), where
            assert np.array_equal(h(sp)[b], rp), where
            assert np.array_equal(h(ss)[b], rs), where
