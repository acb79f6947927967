"""The attention entry point that allocates nothing
(ess_sparse_mla_decode_noalloc: partials in the library's fixed per-device
scratch array) gives exactly what ess_sparse_mla_decode gives with a caller
workspace - outputs, log-sum-exp and the miss rows written to the pool - on
two calls in a row, the second with a smaller input (the array keeps the
first call's contents)."""
import numpy as np
import pytest
import torch

from decode_lightning_indexer_amd import ess
from decode_lightning_indexer_amd.session import HostStore
from synth import gen
from tests.gpu_util import dims, sync, t

pytestmark = pytest.mark.gpu


def _case(rng, B, m, H, L, k, C, p_hit):
    """Selections with hits, misses and designated writers (as the pool
    update lays them out), and the host rows."""
    host = HostStore((B, L, 576))
    host.array[:] = gen.f32_to_bf16_bits(
        rng.standard_normal((B, L, 576)).astype(np.float32) * np.float32(0.5))
    qa = gen.f32_to_bf16_bits(rng.standard_normal((B, m, H, 576)).astype(np.float32)
                              * np.float32(0.1))
    n_sel = rng.integers(k // 2, k + 1, (B, m)).astype(np.int32)
    sel = np.full((B, m, k), -1, np.int32)
    src = np.full((B, m, k), -1, np.int32)
    dst = np.full((B, m, k), -1, np.int32)
    pool = np.zeros((B, C, 576), np.uint16)
    for b in range(B):
        slot_of, free = {}, list(rng.permutation(C))
        for j in range(m):
            pos = rng.permutation(L)[:n_sel[b, j]]
            sel[b, j, :len(pos)] = pos
            for i, p in enumerate(pos.tolist()):
                if p not in slot_of:
                    s, hit = free.pop(), rng.random() < p_hit
                    slot_of[p] = (s, hit)
                    if hit:
                        pool[b, s] = host.array[b, p]
                    else:
                        dst[b, j, i] = s
                s, hit = slot_of[p]
                src[b, j, i] = s if hit else -1
    d = dims(batch=B, mtp=m, ctx_len=L, mla_heads=H, topk=k, pool_slots=C)
    return d, host, qa, sel, src, dst, n_sel, pool


def _both(d, host, qa, sel, src, dst, n_sel, pool):
    B, m, H = d.batch, d.mtp, d.mla_heads
    outs = []
    for noalloc in (True, False):
        pool_t = t(pool)
        out = torch.full((B, m, H, 512), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((B, m, H), float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            ess.ess_sparse_mla_decode_noalloc(d, t(qa), t(sel), t(src), t(dst), t(n_sel),
                                              pool_t, host.dev, out, lse)
        else:
            wsb = ess.ess_workspace_bytes(d)
            ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
            ess.ess_sparse_mla_decode(d, t(qa), t(sel), t(src), t(dst), t(n_sel),
                                      pool_t, host.dev, out, lse, ws, wsb)
        sync()
        outs.append((out, lse, pool_t))
    (o1, l1, p1), (o2, l2, p2) = outs
    assert torch.isfinite(o1).all() and torch.isfinite(l1).all()
    assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(p1, p2)


def test_noalloc_equals_workspace_entry_point_on_two_calls():
    rng = np.random.default_rng(77)
    # First call: 4 requests x 128 heads x 2048 rows (32 chunks of partials,
    # 16.8 MB of the array); second: a smaller one (1 request, 2 tokens,
    # 64 heads, 512 rows) over the first call's leftover partials.
    for shape in ((4, 1, 128, 6000, 2048, 4096, 0.7), (1, 2, 64, 1500, 512, 1100, 0.5)):
        print(f"\n[noalloc] B, m, H, L, k, C, p_hit = {shape}", flush=True)
        case = _case(rng, *shape)
        _both(*case)
        case[1].free()


def test_noalloc_refuses_dims_beyond_its_array():
    # 64 requests x 128 heads need 33.6 MB of partials: refused before
    # anything is enqueued.
    d = dims(batch=64, mtp=1, ctx_len=4096, mla_heads=128, topk=2048, pool_slots=4096)
    P = 0x1000
    with pytest.raises(ess.EssError) as e:
        ess.ess_sparse_mla_decode_noalloc(d, P, P, P, P, P, P, P, P, P)
    assert e.value.status == "out of memory" and "scratch" in str(e.value)
