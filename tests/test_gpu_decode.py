"""Whole decode sequences on the GPU (fill, then steps through
ess_decode_step) against the CPU oracle, placement invariance, dense MLA at
k >= L, and prefetch mode against inline mode."""
import numpy as np
import pytest
import torch

from decode_lightning_indexer_amd import ess
from decode_lightning_indexer_amd.runner import DecodeRunner
from decode_lightning_indexer_amd.session import HostStore, dims_of
from oracle import decode as odecode
from synth import get_workload
from synth.device import LayerInputs
from tests.gpu_util import assert_attn_close, h, lse_close, sync

pytestmark = pytest.mark.gpu


def gpu_sequence(wl, steps=None, mode=ess.ESS_MODE_INLINE, layers=None):
    """Fill + steps on the GPU; per step and layer, every output as numpy."""
    steps = wl.steps if steps is None else steps
    layers = wl.layers if layers is None else layers
    d = dims_of(wl)
    B, m, k, C = wl.batch, wl.mtp, wl.topk, wl.pool_slots
    hosts = [HostStore((B, wl.ctx_len, 576)) for _ in range(layers)]
    ins = [LayerInputs(wl, l) for l in range(layers)]
    run = DecodeRunner(d, hosts)
    for l in range(layers):
        ins[l].upload_static(run.layers[l], hosts[l].array)
    run.set_n_vis(ins[0].n_vis)
    run.reset()
    for l in range(layers):
        ins[l].upload_step(run.layers[l], 0)
    run.fill()
    sync()
    recs = {"fill": [], "steps": []}
    for l, lb in enumerate(run.layers):
        nm = h(lb.n_miss)
        mp = h(lb.lists(lb.miss_pos, C))
        recs["fill"].append(dict(n_miss=nm, miss_pos=mp, miss_slot=h(lb.lists(lb.miss_slot, C))))
    for t in range(steps):
        for l in range(layers):
            ins[l].upload_step(run.layers[l], t)
        run.step(mode)
        sync()
        per = []
        for lb in run.layers:
            per.append(dict(
                sel_pos=h(lb.rows(lb.sel_pos, k, m)), sel_slot=h(lb.rows(lb.sel_slot, k, m)),
                n_sel=h(lb.n_sel), row_dst=h(lb.rows(lb.row_dst, k, m)),
                sel_slot_post=h(lb.rows(lb.sel_slot_post, k, m)),
                miss_pos=h(lb.lists(lb.miss_pos, m * k)), miss_slot=h(lb.lists(lb.miss_slot, m * k)),
                n_miss=h(lb.n_miss), n_evict=h(lb.n_evict), out=h(lb.out), lse=h(lb.lse)))
        recs["steps"].append(per)
    # Every resident slot holds its host row.
    for l, lb in enumerate(run.layers):
        cs, pool = h(lb.cache_slots), h(lb.pool)
        for b in range(B):
            res = np.nonzero(cs[b] >= 0)[0]
            assert np.array_equal(pool[b, cs[b, res]], hosts[l].array[b, res]), (l, b)
    for hst in hosts:
        hst.free()
    return recs


def compare_with_oracle(wl, recs, layer=0, requests=None, steps=None):
    requests = range(wl.batch) if requests is None else requests
    steps = len(recs["steps"]) if steps is None else steps
    worst = 0.0
    for b in requests:
        it = odecode.run_workload_request(wl, layer, b, steps=steps)
        fill = next(it)
        g = recs["fill"][layer]
        n = int(g["n_miss"][b])
        assert n == fill["n_miss"]
        assert np.array_equal(g["miss_pos"][b, :n], fill["miss_pos"])
        assert np.array_equal(g["miss_slot"][b, :n], fill["miss_slot"])
        for t, ref in enumerate(it):
            g = recs["steps"][t][layer]
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


def test_tiny_sequence_matches_oracle():
    wl = get_workload("tiny-4k")
    recs = gpu_sequence(wl)
    compare_with_oracle(wl, recs)
    # Drift produced misses after step 0.
    assert sum(int(s[0]["n_miss"][0]) for s in recs["steps"]) > 0


def test_mtp2_sequence_matches_oracle():
    wl = get_workload("tiny-4k").with_(
        name="mtp2-small", batch=2, mtp=2, ctx_len=8192, idx_heads=64,
        idx_dim=128, mla_heads=32, topk=512, pool_slots=2048, steps=6, rho=0.9)
    recs = gpu_sequence(wl)
    compare_with_oracle(wl, recs)


def test_placement_invariance_all_resident():
    wl = get_workload("tiny-4k").with_(steps=4)
    a = gpu_sequence(wl)
    b = gpu_sequence(wl.with_(pool_slots=wl.ctx_len))
    for sa, sb in zip(a["steps"], b["steps"]):
        assert np.array_equal(sa[0]["sel_pos"], sb[0]["sel_pos"])
        assert int(sb[0]["n_miss"][0]) == 0
        assert np.array_equal(sa[0]["out"], sb[0]["out"])
        assert np.array_equal(sa[0]["lse"], sb[0]["lse"])


def test_k_at_least_context_is_dense():
    wl = get_workload("tiny-4k").with_(ctx_len=1000, topk=2048, pool_slots=4096, steps=2)
    recs = gpu_sequence(wl)
    for s in recs["steps"]:
        assert int(s[0]["n_sel"][0, 0]) == 1000
    compare_with_oracle(wl, recs)


def test_prefetch_mode_equals_inline():
    wl = get_workload("tiny-4k").with_(
        name="3layer", batch=2, layers=3, steps=4, miss_mode="prefetch")
    a = gpu_sequence(wl, mode=ess.ESS_MODE_INLINE)
    b = gpu_sequence(wl, mode=ess.ESS_MODE_PREFETCH)
    for sa, sb in zip(a["steps"], b["steps"]):
        for la, lb in zip(sa, sb):
            for key in la:
                assert np.array_equal(la[key], lb[key]), key
    for layer in range(3):
        compare_with_oracle(wl, b, layer=layer, requests=[1])
