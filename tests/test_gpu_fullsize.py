"""GPU parity at the workloads' real sizes, through the same whole-step entry
point the benchmark drives.  Every request is checked for the properties
that hold at any size (every resident slot holds its host row bit for bit,
inside gpu_sequence); sampled requests are compared with the CPU oracle
element by element: top-k, slot lists, miss lists and counts bit-exact,
attention within tolerance."""
import numpy as np
import pytest

from decode_lightning_indexer_amd import ess
from synth import get_workload
from tests.gpu_util import compare_with_oracle, gpu_sequence

pytestmark = pytest.mark.gpu


def _check(wl, requests, mode=ess.ESS_MODE_INLINE, layers=None, check_layers=None):
    print(f"\n[fullsize] {wl.name}: B={wl.batch} m={wl.mtp} L={wl.ctx_len} "
          f"k={wl.topk} C={wl.pool_slots} steps={wl.steps} mode={mode}", flush=True)
    recs = gpu_sequence(wl, mode=mode, layers=layers)
    n_layers = wl.layers if layers is None else layers
    for layer in (range(n_layers) if check_layers is None else check_layers):
        compare_with_oracle(wl, recs, layer=layer, requests=requests)
    misses = sum(int(s[0]["n_miss"].sum()) for s in recs["steps"][1:])
    assert misses > 0, "drift should produce misses after the first step"
    return recs


def test_32k_b16_full_size():
    wl = get_workload("32k-b16").with_(steps=4)
    _check(wl, requests=[0, 15])


def test_128k_b8_mtp2_full_size():
    wl = get_workload("128k-b8-mtp2-r095").with_(steps=4)
    recs = _check(wl, requests=[0, 7])
    # Both MTP ways select their own rows.
    assert np.all(recs["steps"][-1][0]["n_sel"] == wl.topk)


def test_128k_b8_mtp2_heavy_misses_full_size():
    # About half of every step's selection misses: the LRU ring turns over
    # fast (victim scans over dead entries, compaction when it fills).
    wl = get_workload("128k-b8-mtp2-r080").with_(steps=3)
    recs = _check(wl, requests=[3])
    n_miss = sum(int(s[0]["n_miss"].sum()) for s in recs["steps"][1:])
    assert n_miss > 0.3 * 2 * wl.batch * wl.mtp * wl.topk


def test_1m_b1_c16k_full_size():
    wl = get_workload("1m-b1-c16k").with_(steps=4)
    _check(wl, requests=[0])


def test_1m_b1_c8k_full_size():
    wl = get_workload("1m-b1-c8k").with_(steps=3)
    _check(wl, requests=[0])


def test_64k_b32_two_layers_prefetch_full_size():
    # Two of the sixteen layers at full per-layer size (32 requests x 64K
    # positions each), in the side-stream prefetch mode.
    wl = get_workload("64k-b32-16layer").with_(steps=3)
    _check(wl, requests=[0, 31], mode=ess.ESS_MODE_PREFETCH, layers=2)


def test_64k_b32_sixteen_layers_prefetch_full_size():
    # All sixteen layers (38.7 GB of host latents, each layer its own pool and
    # seeds) selected ahead on the side stream; the first, a middle and the
    # last layer against the oracle on one request.
    wl = get_workload("64k-b32-16layer").with_(steps=2)
    _check(wl, requests=[5], mode=ess.ESS_MODE_PREFETCH, check_layers=[0, 7, 15])


def test_32k_b16_fp8_entries_full_size():
    # The host store as 656-byte fp8 entries at full size: the oracle runs
    # on the dequantized latents.
    from tests.gpu_util import dequantized_latents
    wl = get_workload("32k-b16").with_(steps=3)
    print(f"\n[fullsize] {wl.name} fp8 entries", flush=True)
    recs = gpu_sequence(wl, store="entries")
    _, eff = dequantized_latents(wl, 0)
    compare_with_oracle(wl, recs, requests=[0, 15], host=eff)


def test_32k_b16_growing_context_full_size():
    # Four steps of growth that cross a 64-token block boundary (a block
    # written back mid-run), at the full 32K x 16 shape.
    from tests.test_gpu_growth import _grow
    wl = get_workload("32k-b16").with_(steps=4)
    L0 = 32702
    print(f"\n[fullsize] {wl.name} growing from {L0}", flush=True)
    recs, _ = _grow(wl, L0, 64, ess.ESS_MODE_INLINE, 4)
    compare_with_oracle(wl, recs, requests=[0, 15], grow_from=L0)
