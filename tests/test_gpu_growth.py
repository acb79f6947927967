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
from oracle.formats import encode_entries as oracle_encode_entries
from tests.gpu_util import compare_with_oracle, dequantized_latents, h, sync

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0


def _grow(wl, L0, block, mode, steps, layers=1, store="bf16"):
    """L0: the initial length, one per request or one for all.  store:
    "bf16" rows or 656-byte fp8 "entries" (then every latent the path sees
    is the dequantized entry, and the oracle runs on those)."""
    B, m, L, k = wl.batch, wl.mtp, wl.ctx_len, wl.topk
    d = dims_of(wl)
    L0 = list(L0) if isinstance(L0, (list, tuple)) else [L0] * B
    lats, keys, hosts, ents, effs = [], [], [], [], []
    for l in range(layers):
        lat = np.empty((B, L, 576), np.uint16)
        gen.fill_latents(wl, l, lat)
        kb = np.empty((B, L, wl.idx_dim), np.uint8)
        gen.fill_index_keys(wl, l, kb)
        if store == "bf16":
            host = HostStore((B, L, 576))
            host.array[:] = NAN_BF16
            for b in range(B):
                host.array[b, :L0[b]] = lat[b, :L0[b]]
            effs.append(lat)
        else:
            ent, eff = dequantized_latents(wl, l)
            host = HostStore((B, L, 656), np.uint8)
            host.array[:] = 0x7F                     # NaN codes and NaN scales
            for b in range(B):
                host.array[b, :L0[b]] = ent[b, :L0[b]]
            ents.append(ent)
            effs.append(eff)
        lats.append(lat); keys.append(kb); hosts.append(host)
    if store == "bf16":
        run = DecodeRunner(d, hosts)
    else:
        run = DecodeRunner(d, [None] * layers, entries=hosts)
    ins = [LayerInputs(wl, l) for l in range(layers)]
    for l, lb in enumerate(run.layers):
        ins[l].upload_static(lb, None, keys=False, latents=False)
        k0 = np.zeros_like(keys[l])
        for b in range(B):
            k0[b, :L0[b]] = keys[l][b, :L0[b]]
        lb.k_idx.copy_(torch.from_numpy(k0))
        ins[l].upload_step(lb, 0)
    run.set_n_vis([[L0[b] - m + 1 + j for j in range(m)] for b in range(B)])
    run.reset()
    run.fill()
    sync()
    recs = {"fill": [dict(n_miss=h(lb.n_miss), miss_pos=h(lb.lists(lb.miss_pos, wl.pool_slots)),
                          miss_slot=h(lb.lists(lb.miss_slot, wl.pool_slots)))
                     for lb in run.layers], "steps": []}
    stream = torch.cuda.current_stream()
    d2h = torch.cuda.Stream()
    rows, states, tails, new_keys, new_lat, tail_ents = [], [], [], [], [], []
    for l in range(layers):
        rows.append(torch.full((B, 2 * block, 576), NAN_BF16, dtype=torch.int16, device="cuda"))
        states.append(torch.empty(3 * B, dtype=torch.int32, device="cuda"))
        tail_ents.append(None if store == "bf16" else
                         torch.full((B, 2 * block, 656), 0x7F, dtype=torch.uint8, device="cuda"))
        tails.append(ess.ess_tail_init(d, rows[l], block, L0, states[l], stream,
                                       entries=tail_ents[l]))
        # Each request's new tokens, [steps][B][m][...].
        new_keys.append(torch.from_numpy(np.ascontiguousarray(np.stack(
            [keys[l][b, L0[b]:L0[b] + steps * m].reshape(steps, m, -1) for b in range(B)], 1))).cuda())
        new_lat.append(torch.from_numpy(np.ascontiguousarray(np.stack(
            [lats[l][b, L0[b]:L0[b] + steps * m].reshape(steps, m, 576) for b in range(B)],
            1)).view(np.int16)).cuda())
    # Every layer's n_vis is the same; each layer's append writes it again.
    from_tail = 0
    for t in range(steps):
        ios = []
        for l, lb in enumerate(run.layers):
            ins[l].upload_step(lb, t)
            ess.ess_append_tokens(d, tails[l], new_keys[l][t], new_lat[l][t], lb.k_idx,
                                  run.n_vis, hosts[l].host, stream, d2h)
            io = lb.io()
            io.tail_rows, io.tail_start, io.tail_block = (rows[l].data_ptr(), tails[l].start_dev,
                                                          block)
            ios.append(io)
        ess.ess_decode_step(d, ios, run.n_vis, mode, stream, run.side)
        sync()
        per = []
        for l, lb in enumerate(run.layers):
            nm = h(lb.n_miss)
            mp = h(lb.lists(lb.miss_pos, m * k))
            st = tails[l].start
            assert h(states[l]).tolist() == tails[l].first + tails[l].n_ctx + st
            from_tail += sum(int((mp[b, :nm[b]] >= st[b]).sum()) for b in range(B))
            per.append(dict(
                sel_pos=h(lb.rows(lb.sel_pos, k, m)), sel_slot=h(lb.rows(lb.sel_slot, k, m)),
                n_sel=h(lb.n_sel), row_dst=h(lb.rows(lb.row_dst, k, m)),
                sel_slot_post=h(lb.rows(lb.sel_slot_post, k, m)),
                miss_pos=mp, miss_slot=h(lb.lists(lb.miss_slot, m * k)),
                n_miss=nm, n_evict=h(lb.n_evict), out=h(lb.out), lse=h(lb.lse)))
        recs["steps"].append(per)
    torch.cuda.synchronize()
    for l, lb in enumerate(run.layers):
        assert tails[l].n_ctx == [L0[b] + steps * m for b in range(B)]
        for b in range(B):
            # Written back: every full block from L0 on; beyond it the host
            # store is untouched.  Entries written back are the oracle's
            # quantization of the latents.
            done = ((L0[b] + steps * m) // block) * block
            if store == "bf16":
                assert np.array_equal(hosts[l].array[b, :done], lats[l][b, :done]), (l, b)
                assert np.all(hosts[l].array[b, max(done, L0[b]):] == NAN_BF16), (l, b)
            else:
                assert np.array_equal(hosts[l].array[b, :L0[b]], ents[l][b, :L0[b]]), (l, b)
                assert np.array_equal(hosts[l].array[b, L0[b]:done],
                                      oracle_encode_entries(lats[l][b, L0[b]:done])), (l, b)
                assert np.all(hosts[l].array[b, max(done, L0[b]):] == 0x7F), (l, b)
        # Every resident slot holds its latent, wherever it came from.
        cs, pool = h(lb.cache_slots), h(lb.pool)
        for b in range(B):
            res = np.nonzero(cs[b] >= 0)[0]
            assert np.array_equal(pool[b, cs[b, res]], effs[l][b, res]), (l, b)
        ess.ess_tail_release(tails[l])
        hosts[l].free()
    if store != "bf16":
        recs["effective"] = effs
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


def test_growth_two_layers_prefetch():
    # Two layers, each with its own tail and host store, selected ahead on
    # the side stream: every layer against the oracle.
    steps, m, block = 12, 2, 8
    wl = get_workload("tiny-4k").with_(name="grow2", batch=2, mtp=m, ctx_len=2048,
                                       topk=256, pool_slots=1024, steps=steps, rho=0.9,
                                       layers=2)
    L0 = 2048 - steps * m - 3
    print(f"growth two layers m={m} block={block} L0={L0}", flush=True)
    recs, from_tail = _grow(wl, L0, block, ess.ESS_MODE_PREFETCH, steps, layers=2)
    assert from_tail > 0
    for layer in range(2):
        compare_with_oracle(wl, recs, layer=layer, grow_from=L0)


def test_growth_requests_at_different_lengths():
    # Four requests starting at different lengths (block boundaries, and so
    # write-backs, fall on different steps for each).
    steps, m, block = 20, 2, 8
    wl = get_workload("tiny-4k").with_(name="grow-ragged", batch=4, mtp=m, ctx_len=2048,
                                       topk=256, pool_slots=1024, steps=steps, rho=0.9)
    L0 = [1500, 1733, 2048 - steps * m, 901]
    print(f"growth ragged lengths {L0} m={m} block={block}", flush=True)
    recs, from_tail = _grow(wl, L0, block, ess.ESS_MODE_INLINE, steps)
    assert from_tail > 0
    compare_with_oracle(wl, recs, grow_from=L0)


@pytest.mark.parametrize("mode", [ess.ESS_MODE_INLINE, ess.ESS_MODE_PREFETCH])
def test_growth_over_fp8_entries(mode):
    # A host store of fp8 entries: appended tokens are quantized on the GPU,
    # written back as entries (bit-exact against the oracle's quantizer) and
    # read from the tail as the dequantized entry; requests at different
    # lengths, blocks of 6 tokens.
    steps, m, block = 16, 2, 6
    wl = get_workload("tiny-4k").with_(name="grow-fp8", batch=3, mtp=m, ctx_len=2048,
                                       topk=256, pool_slots=1024, steps=steps, rho=0.9)
    L0 = [1990, 1601, 1777]
    print(f"growth over entries mode={mode} lengths {L0} block={block}", flush=True)
    recs, from_tail = _grow(wl, L0, block, mode, steps, store="entries")
    assert from_tail > 0
    compare_with_oracle(wl, recs, grow_from=L0, host=recs["effective"][0])
