"""Whole decode sequences on the GPU (fill, then steps through
ess_decode_step) against the CPU oracle, placement invariance, dense MLA at
k >= L, and prefetch mode against inline mode."""
import numpy as np
import pytest
import torch

from decode_lightning_indexer_amd import ess
from synth import get_workload
from tests.gpu_util import compare_with_oracle, gpu_sequence

pytestmark = pytest.mark.gpu


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


@pytest.mark.parametrize("m,k", [(3, 512), (4, 256)])
def test_three_and_four_tokens_match_oracle(m, k):
    # More than two query tokens per request: the residency update merges
    # the tokens' position lists by searches in the other lists (two tokens
    # take a merge path).
    wl = get_workload("tiny-4k").with_(
        name=f"mtp{m}-small", batch=2, mtp=m, ctx_len=8192, idx_heads=32,
        idx_dim=128, mla_heads=32, topk=k, pool_slots=2048, steps=5, rho=0.9)
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


def test_long_rows_fill_and_steps_select_in_levels():
    # 50K positions with C = 3000 and k = 512: the first fill's top-C and every
    # step's top-k run the multi-level selection (rows over 32768 keys, k and
    # C <= 4096), for two requests with two MTP ways each.
    wl = get_workload("tiny-4k").with_(
        name="long-levels", batch=2, mtp=2, ctx_len=50000, idx_heads=16,
        idx_dim=64, mla_heads=16, topk=512, pool_slots=3000, steps=3, rho=0.9)
    recs = gpu_sequence(wl)
    compare_with_oracle(wl, recs)


def test_lru_replay_reproduces_the_gpu_pool():
    # The host replay of the recorded steps (ess_replay_evictions, LRU, the
    # workload's pool size) gives the GPU pool update's miss count at every
    # request and step; Score and Random replays of the same trace stay
    # within the union of each step.
    from decode_lightning_indexer_amd.runner import DecodeRunner
    from decode_lightning_indexer_amd.session import HostStore, dims_of
    from synth.device import LayerInputs
    wl = get_workload("tiny-4k").with_(
        name="replay", batch=3, mtp=2, ctx_len=6000, idx_heads=32, idx_dim=128,
        mla_heads=16, topk=256, pool_slots=700, steps=8, rho=0.85)
    B, m, k, T = wl.batch, wl.mtp, wl.topk, wl.steps
    host = HostStore((B, wl.ctx_len, 576))
    ins = LayerInputs(wl, 0)
    run = DecodeRunner(dims_of(wl), [host])
    lb = run.layers[0]
    ins.upload_static(lb, host.array)
    run.set_n_vis(ins.n_vis)
    run.reset()
    ins.upload_step(lb, 0)
    run.fill()
    scores = np.empty((B, T, m, wl.ctx_len), np.float32)
    sel = np.empty((B, T, m, k), np.int32)
    n_sel = np.empty((B, T, m), np.int32)
    gpu = np.empty((B, T), np.int32)
    for t in range(T):
        ins.upload_step(lb, t)
        run.step(ess.ESS_MODE_INLINE)
        torch.cuda.synchronize()
        scores[:, t] = lb.scores.cpu().numpy()
        sel[:, t] = lb.rows(lb.sel_pos, k, m).cpu().numpy()
        n_sel[:, t] = lb.n_sel.cpu().numpy()
        gpu[:, t] = lb.n_miss.cpu().numpy()
    host.free()
    assert gpu[:, 1:].sum() > 0
    for b in range(B):
        nm, _ = ess.ess_replay_evictions(ess.ESS_EVICT_LRU, wl.pool_slots,
                                         scores[b], sel[b], n_sel[b], request=b)
        assert np.array_equal(nm, gpu[b]), b
        for pol in (ess.ESS_EVICT_RANDOM, ess.ESS_EVICT_SCORE):
            nm2, ev2 = ess.ess_replay_evictions(pol, wl.pool_slots, scores[b],
                                                sel[b], n_sel[b], request=b)
            assert np.all(ev2 <= nm2) and np.all(nm2 <= m * k)


def test_concurrent_sequences_on_two_threads():
    # Two host threads run whole prefetch-mode sequences at once (each with
    # its own buffers and side stream; the library's stream-ordering events
    # are per thread): both equal the same sequences run one after another.
    import threading
    wls = [get_workload("tiny-4k").with_(name=f"thread{i}", batch=2, layers=2,
                                          steps=3, seed=11 + i, miss_mode="prefetch")
           for i in range(2)]
    ref = [gpu_sequence(wl, mode=ess.ESS_MODE_PREFETCH) for wl in wls]
    got = [None, None]
    errs = []

    def work(i):
        try:
            got[i] = gpu_sequence(wls[i], mode=ess.ESS_MODE_PREFETCH)
        except Exception as e:          # surfaced below
            errs.append(e)

    th = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    assert not errs, errs
    for i in range(2):
        for sa, sb in zip(ref[i]["steps"], got[i]["steps"]):
            for la, lb in zip(sa, sb):
                for key in la:
                    assert np.array_equal(la[key], lb[key]), (i, key)
