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
