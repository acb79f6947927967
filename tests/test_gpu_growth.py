"""Growing context on the GPU: every step appends its tokens through
ess_append_tokens (keys to the index cache, latents to the tail blocks, full
blocks written back to the host store) and runs ess_decode_step with the tail
view.  Against the oracle run on the same growth; the host store holds every
written-back block bit for bit and nothing past it (it starts as NaN there,
so a read of a position before its write-back would show)."""
import numpy as np
import pytest
import torch

from decode_lightning_indexer_amd import ess
from decode_lightning_indexer_amd.runner import DecodeRunner
from decode_lightning_indexer_amd.session import HostStore, dims_of
from synth import gen, get_workload
from synth.device import LayerInputs
from tests.gpu_util import compare_with_oracle, h, sync

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0


def _grow(wl, L0, block, mode, steps):
    B, m, L, k = wl.batch, wl.mtp, wl.ctx_len, wl.topk
    d = dims_of(wl)
    lat = np.empty((B, L, 576), np.uint16)
    gen.fill_latents(wl, 0, lat)
    keys = np.empty((B, L, wl.idx_dim), np.uint8)
    gen.fill_index_keys(wl, 0, keys)
    host = HostStore((B, L, 576))
    host.array[:] = NAN_BF16
    host.array[:, :L0] = lat[:, :L0]
    run = DecodeRunner(d, [host])
    lb = run.layers[0]
    ins = LayerInputs(wl, 0)
    ins.upload_static(lb, None, keys=False, latents=False)
    k0 = np.zeros_like(keys)
    k0[:, :L0] = keys[:, :L0]
    lb.k_idx.copy_(torch.from_numpy(k0))
    run.set_n_vis([[L0 - m + 1 + j for j in range(m)]] * B)
    run.reset()
    ins.upload_step(lb, 0)
    run.fill()
    sync()
    recs = {"fill": [dict(n_miss=h(lb.n_miss), miss_pos=h(lb.lists(lb.miss_pos, wl.pool_slots)),
                          miss_slot=h(lb.lists(lb.miss_slot, wl.pool_slots)))], "steps": []}
    rows = torch.full((B, 2 * block, 576), NAN_BF16, dtype=torch.int16, device="cuda")
    tail = ess.ess_tail_init(rows, block, L0)
    stream = torch.cuda.current_stream()
    d2h = torch.cuda.Stream()
    new_keys = torch.from_numpy(np.ascontiguousarray(keys[:, L0:L0 + steps * m])).cuda()
    new_lat = torch.from_numpy(np.ascontiguousarray(lat[:, L0:L0 + steps * m]).view(np.int16)).cuda()
    from_tail = 0
    for t in range(steps):
        ins.upload_step(lb, t)
        ess.ess_append_tokens(d, tail, new_keys[:, t * m:(t + 1) * m].contiguous(),
                              new_lat[:, t * m:(t + 1) * m].contiguous(), lb.k_idx,
                              run.n_vis, host.host, stream, d2h)
        io = lb.io()
        io.tail_rows, io.tail_start, io.tail_block = rows.data_ptr(), tail.start, block
        ess.ess_decode_step(d, [io], run.n_vis, mode, stream, run.side)
        sync()
        nm = h(lb.n_miss)
        mp = h(lb.lists(lb.miss_pos, m * k))
        from_tail += sum(int((mp[b, :nm[b]] >= tail.start).sum()) for b in range(B))
        recs["steps"].append([dict(
            sel_pos=h(lb.rows(lb.sel_pos, k, m)), sel_slot=h(lb.rows(lb.sel_slot, k, m)),
            n_sel=h(lb.n_sel), row_dst=h(lb.rows(lb.row_dst, k, m)),
            sel_slot_post=h(lb.rows(lb.sel_slot_post, k, m)),
            miss_pos=mp, miss_slot=h(lb.lists(lb.miss_slot, m * k)),
            n_miss=nm, n_evict=h(lb.n_evict), out=h(lb.out), lse=h(lb.lse))])
    torch.cuda.synchronize()
    n_ctx = L0 + steps * m
    assert tail.n_ctx == n_ctx
    # Written back: every full block from L0 on; beyond it the host store is untouched.
    done = (n_ctx // block) * block
    assert np.array_equal(host.array[:, :done], lat[:, :done])
    assert np.all(host.array[:, max(done, L0):] == NAN_BF16)
    # Every resident slot holds its latent, wherever it came from.
    cs, pool = h(lb.cache_slots), h(lb.pool)
    for b in range(B):
        res = np.nonzero(cs[b] >= 0)[0]
        assert np.array_equal(pool[b, cs[b, res]], lat[b, res]), b
    ess.ess_tail_release(tail)
    host.free()
    return recs, from_tail


@pytest.mark.parametrize("mode", [ess.ESS_MODE_INLINE, ess.ESS_MODE_PREFETCH])
@pytest.mark.parametrize("m,block", [(1, 16), (2, 8), (2, 5)])
def test_growth_matches_oracle(mode, m, block):
    steps = 24
    wl = get_workload("tiny-4k").with_(name="grow", batch=2, mtp=m, ctx_len=2048,
                                       topk=256, pool_slots=1024, steps=steps, rho=0.9)
    L0 = 2048 - steps * m - 7
    print(f"growth mode={mode} m={m} block={block} L0={L0}", flush=True)
    recs, from_tail = _grow(wl, L0, block, mode, steps)
    assert from_tail > 0               # some misses were served from the tail
    compare_with_oracle(wl, recs, grow_from=L0)
