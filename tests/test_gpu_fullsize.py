"""GPU parity at the workloads' real sizes, through the same whole-step entry
point the benchmark drives, over every step of each workload.  Every request
is checked for the properties that hold at any size (every resident slot
holds its host row bit for bit, inside gpu_sequence; the pool state reports
no inconsistency); sampled requests are compared with the CPU oracle element
by element at every step: top-k, slot lists, miss lists and counts
bit-exact, attention within tolerance, and for one request per workload its
whole score rows bit-exact.

The recency ring of a request holds 4C entries and each update pushes its
union (k entries per token way), so it first compacts after
(4C - C) / |union| updates.  Where a workload's own step count stops short
of that (1M: 12 and 24 steps; 64K x 16 layers: 24 steps), the run goes on
until the ring has compacted, and the compaction is asserted from the pool
status."""
import numpy as np
import pytest

from decode_lightning_indexer_amd import ess
from synth import get_workload
from tests.gpu_util import compare_with_oracle, gpu_sequence

pytestmark = pytest.mark.gpu


def _steps_to_compact(wl):
    """Updates after the fill until the ring first compacts (union = m*k at
    most; the ring is compacted when a push would overflow it)."""
    cap, fill, per = 4 * wl.pool_slots, wl.pool_slots, wl.topk
    return (cap - fill) // per + 1


def _check(wl, requests, mode=ess.ESS_MODE_INLINE, layers=None, check_layers=None,
           score_request=None, expect_compaction=True):
    n_layers = wl.layers if layers is None else layers
    check_layers = list(range(n_layers)) if check_layers is None else list(check_layers)
    score_request = requests[0] if score_request is None else score_request
    print(f"\n[fullsize] {wl.name}: B={wl.batch} m={wl.mtp} L={wl.ctx_len} "
          f"k={wl.topk} C={wl.pool_slots} steps={wl.steps} layers={n_layers} "
          f"mode={mode} requests={requests}", flush=True)
    recs = gpu_sequence(wl, mode=mode, layers=layers, keep=requests,
                        keep_layers=check_layers, score_requests=[score_request])
    for layer in check_layers:
        compare_with_oracle(wl, recs, layer=layer, requests=requests)
        print(f"[fullsize] {wl.name} layer {layer}: {wl.steps} steps exact", flush=True)
    for layer, st in enumerate(recs["status"]):
        assert (st[:, 0] == 0).all(), (layer, st[:, 0])          # no error flag
        assert (st[:, 2] == wl.steps + 1).all(), (layer, st[:, 2])   # fill + steps
        if expect_compaction:
            assert (st[:, 1] >= 1).all(), (layer, st[:, 1])
    misses = sum(int(s[check_layers[0]]["n_miss"].sum()) for s in recs["steps"][1:])
    assert misses > 0, "drift should produce misses after the first step"
    return recs


def test_32k_b16_full_size():
    wl = get_workload("32k-b16")
    assert wl.steps >= _steps_to_compact(wl)
    _check(wl, requests=[0, 5, 10, 15])


@pytest.mark.parametrize("name", ["128k-b8-mtp2-r099", "128k-b8-mtp2-r095",
                                  "128k-b8-mtp2-r080"])
def test_128k_b8_mtp2_full_size(name):
    wl = get_workload(name)
    recs = _check(wl, requests=[0, 7])
    # Both MTP ways select their own rows.
    assert np.all(recs["steps"][-1][0]["n_sel"] == wl.topk)
    if name.endswith("r080"):
        # About half of every step's selection misses: the ring turns over
        # fast (victim scans over dead entries, compaction when it fills).
        n_miss = sum(int(s[0]["n_miss"].sum()) for s in recs["steps"][1:])
        assert n_miss > 0.3 * (wl.steps - 1) * wl.batch * wl.mtp * wl.topk


@pytest.mark.parametrize("name", ["1m-b1-c8k", "1m-b1-c16k"])
def test_1m_b1_full_size(name):
    base = get_workload(name)
    wl = base.with_(steps=max(base.steps, _steps_to_compact(base)))
    _check(wl, requests=[0])


def test_64k_b32_sixteen_layers_prefetch_full_size():
    # All sixteen layers (38.7 GB of host latents, each layer its own pool and
    # seeds) selected ahead on the side stream; every layer against the
    # oracle on the first and last requests.
    base = get_workload("64k-b32-16layer")
    wl = base.with_(steps=max(base.steps, _steps_to_compact(base)))
    _check(wl, requests=[0, 31], mode=ess.ESS_MODE_PREFETCH)


def test_64k_b32_two_layers_inline_full_size():
    # Two layers at full per-layer size run inline (each layer selected, then
    # attended, on one stream).
    wl = get_workload("64k-b32-16layer").with_(steps=3)
    _check(wl, requests=[3, 28], layers=2, expect_compaction=False)


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
