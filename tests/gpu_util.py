"""Helpers shared by the GPU parity tests."""
import numpy as np
import torch

from decode_lightning_indexer_amd import ess
from decode_lightning_indexer_amd.runner import DecodeRunner
from decode_lightning_indexer_amd.session import HostStore, dims_of
from oracle import decode as odecode
from oracle.formats import decode_entries
from synth import gen
from synth.device import LayerInputs

DEV = "cuda"

# Attention tolerance: max |d| <= 1e-2 * max |ref| and sum |d| / sum |ref|
# <= 2e-3 over all outputs of a step.
MAX_ABS_REL = 1e-2
MEAN_REL = 2e-3


def attn_errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = np.abs(got - ref)
    return d.max() / np.abs(ref).max(), d.sum() / np.abs(ref).sum()


def assert_attn_close(got, ref, what=""):
    mx, mean = attn_errors(got, ref)
    assert mx <= MAX_ABS_REL and mean <= MEAN_REL, (what, mx, mean)
    return mx, mean


def lse_close(got, ref, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.abs(got - ref).max() <= 1e-3 * max(1.0, np.abs(ref).max()), what


def t(x, dtype=None):
    """numpy -> device tensor (uint16 arrays travel as int16)."""
    a = np.ascontiguousarray(x)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    tt = torch.from_numpy(a)
    if dtype is not None:
        tt = tt.to(dtype)
    return tt.to(DEV)


def h(x):
    """device tensor -> numpy (int16 -> uint16 bits)."""
    a = x.detach().cpu().numpy()
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    return a


def sync():
    torch.cuda.synchronize()


def dims(**kw):
    base = dict(batch=1, mtp=1, ctx_len=1024, idx_heads=16, idx_dim=64,
                mla_heads=16, topk=64, pool_slots=256, softmax_scale=1 / 24)
    base.update(kw)
    return ess.make_dims(**base)


def dequantized_latents(wl, layer):
    """(entries [B][L][656], their dequantized latents [B][L][576] as bf16
    bits) of a layer's generated latents."""
    from concurrent.futures import ThreadPoolExecutor
    B, L = wl.batch, wl.ctx_len
    ent = np.empty((B, L, 656), np.uint8)
    eff = np.empty((B, L, 576), np.uint16)

    def one(b):
        ent[b] = gen.encode_entries(gen.latents(wl, layer, b))
        eff[b] = gen.f32_to_bf16_bits(decode_entries(ent[b]).astype(np.float32))
    with ThreadPoolExecutor(max_workers=8) as ex:
        list(ex.map(one, range(B)))
    return ent, eff


def gpu_sequence(wl, steps=None, mode=ess.ESS_MODE_INLINE, layers=None,
                 store="bf16", keep=None, keep_layers=None, score_requests=()):
    """Fill + steps on the GPU; per step and layer, every output as numpy.
    store: "bf16" (generated latents as bf16 rows), "entries" (656-byte fp8
    entries of them) or "dequantized" (bf16 rows of the dequantized
    entries).  keep: the requests whose outputs are recorded (all if None;
    arrays keep the request axis, other requests' rows are zero);
    keep_layers: the layers recorded (all if None); score_requests: requests
    whose whole score rows are recorded every step.  recs["status"][l] is
    the layer's ess_pool_status after the last step."""
    steps = wl.steps if steps is None else steps
    layers = wl.layers if layers is None else layers
    d = dims_of(wl)
    B, m, k, C = wl.batch, wl.mtp, wl.topk, wl.pool_slots
    ins = [LayerInputs(wl, l) for l in range(layers)]
    hosts, entries, rows = [], [], []
    for l in range(layers):
        if store == "bf16":
            hosts.append(HostStore((B, wl.ctx_len, 576)))
            entries.append(None)
            continue
        ent, eff = dequantized_latents(wl, l)
        rows.append(eff)
        if store == "entries":
            hosts.append(None)
            entries.append(HostStore((B, wl.ctx_len, 656), np.uint8))
            entries[-1].array[:] = ent
        else:
            hosts.append(HostStore((B, wl.ctx_len, 576)))
            hosts[-1].array[:] = eff
            entries.append(None)
    run = DecodeRunner(d, hosts, entries=entries)
    for l in range(layers):
        if store == "bf16":
            ins[l].upload_static(run.layers[l], hosts[l].array)
            rows.append(hosts[l].array)
        else:
            ins[l].upload_static(run.layers[l], None, latents=False)
    run.set_n_vis(ins[0].n_vis)
    run.reset()
    for l in range(layers):
        ins[l].upload_step(run.layers[l], 0)
    run.fill()
    sync()
    recs = {"fill": [], "steps": [], "status": []}
    for l, lb in enumerate(run.layers):
        nm = h(lb.n_miss)
        mp = h(lb.lists(lb.miss_pos, C))
        recs["fill"].append(dict(n_miss=nm, miss_pos=mp, miss_slot=h(lb.lists(lb.miss_slot, C))))
    kept = list(range(B)) if keep is None else list(keep)
    kl = set(range(layers)) if keep_layers is None else set(keep_layers)

    def rec(x):
        a = h(x)
        if keep is None:
            return a
        r = np.zeros_like(a)
        r[kept] = a[kept]
        return r
    for t in range(steps):
        for l in range(layers):
            ins[l].upload_step(run.layers[l], t)
        run.step(mode)
        sync()
        per = []
        for l, lb in enumerate(run.layers):
            if l not in kl:
                per.append(None)
                continue
            per.append(dict(
                sel_pos=rec(lb.rows(lb.sel_pos, k, m)), sel_slot=rec(lb.rows(lb.sel_slot, k, m)),
                n_sel=h(lb.n_sel), row_dst=rec(lb.rows(lb.row_dst, k, m)),
                sel_slot_post=rec(lb.rows(lb.sel_slot_post, k, m)),
                miss_pos=rec(lb.lists(lb.miss_pos, m * k)), miss_slot=rec(lb.lists(lb.miss_slot, m * k)),
                n_miss=h(lb.n_miss), n_evict=h(lb.n_evict), out=rec(lb.out), lse=rec(lb.lse),
                scores={b: h(lb.scores[b]) for b in score_requests}))
        recs["steps"].append(per)
    for lb in run.layers:
        st = torch.empty((B, 4), dtype=torch.int32, device=DEV)
        ess.ess_pool_status(d, lb.lru, st)
        sync()
        recs["status"].append(h(st))
    # Every resident slot holds its host row.
    for l, lb in enumerate(run.layers):
        cs, pool = h(lb.cache_slots), h(lb.pool)
        for b in range(B):
            res = np.nonzero(cs[b] >= 0)[0]
            assert np.array_equal(pool[b, cs[b, res]], rows[l][b, res]), (l, b)
    for hst in hosts + entries:
        if hst is not None:
            hst.free()
    return recs


def compare_with_oracle(wl, recs, layer=0, requests=None, steps=None,
                        host=None, grow_from=None):
    """host: the layer's latents [B][L][576] when they are not the generated
    ones (a store of fp8 entries: their dequantized rows); grow_from: the
    initial context length of a growing run (one per request, or one for
    all)."""
    requests = range(wl.batch) if requests is None else requests
    steps = len(recs["steps"]) if steps is None else steps
    worst = 0.0
    for b in requests:
        want_scores = b in recs["steps"][0][layer].get("scores", {})
        it = odecode.run_workload_request(
            wl, layer, b, steps=steps, host=None if host is None else host[b],
            grow_from=grow_from[b] if isinstance(grow_from, (list, tuple)) else grow_from,
            keep_scores=want_scores)
        fill = next(it)
        g = recs["fill"][layer]
        n = int(g["n_miss"][b])
        assert n == fill["n_miss"]
        assert np.array_equal(g["miss_pos"][b, :n], fill["miss_pos"])
        assert np.array_equal(g["miss_slot"][b, :n], fill["miss_slot"])
        for t, ref in enumerate(it):
            g = recs["steps"][t][layer]
            if want_scores:
                # Whole score rows, bit for bit (-inf past n_vis included).
                assert np.array_equal(g["scores"][b].astype(np.float64), ref["scores"]), (b, t)
            for key in ("sel_pos", "sel_slot", "n_sel", "row_dst", "sel_slot_post"):
                assert np.array_equal(g[key][b], ref[key]), (key, b, t)
            n = int(g["n_miss"][b])
            assert n == ref["n_miss"] and int(g["n_evict"][b]) == ref["n_evict"], (b, t)
            assert np.array_equal(g["miss_pos"][b, :n], ref["miss_pos"]), (b, t)
            assert np.array_equal(g["miss_slot"][b, :n], ref["miss_slot"]), (b, t)
            mx, _ = assert_attn_close(g["out"][b], ref["out"], (b, t))
            lse_close(g["lse"][b], ref["lse"], (b, t))
            worst = max(worst, mx)
    return worst


