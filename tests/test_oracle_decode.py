"""Pins for the oracle's whole decode sequence on the tiny workload: every
step's invariants (asserted inside the driver), placement invariance (an
all-resident pool gives the same selections and outputs), and the pages'
byte arithmetic."""
import numpy as np

from oracle import decode, footprint
from synth import get_workload
from tests.golden.load import load


def _run(wl, steps=None):
    return list(decode.run_workload_request(wl, 0, 0, steps=steps))


def test_tiny_sequence_runs_with_invariants():
    wl = get_workload("tiny-4k")
    recs = _run(wl)
    fill = recs[0]
    assert fill["kind"] == "fill" and fill["n_miss"] == wl.pool_slots
    assert fill["miss_slot"].tolist() == list(range(wl.pool_slots))
    assert np.all(np.diff(fill["miss_pos"]) > 0)
    steps = recs[1:]
    assert len(steps) == wl.steps
    for r in steps:
        assert r["n_sel"].tolist() == [wl.topk]
        assert r["n_evict"] == r["n_miss"]        # pool full after the fill
    # Step 0 uses the same query as the fill, whose selection is a superset.
    assert steps[0]["n_miss"] == 0
    # Drift makes later steps miss some entries.
    assert sum(r["n_miss"] for r in steps) > 0


def test_placement_invariance_all_resident():
    wl = get_workload("tiny-4k").with_(steps=4)
    a = _run(wl)
    b = _run(wl.with_(pool_slots=wl.ctx_len))
    for ra, rb in zip(a[1:], b[1:]):
        assert np.array_equal(ra["sel_pos"], rb["sel_pos"])
        assert rb["n_miss"] == 0
        assert np.array_equal(ra["out"], rb["out"])
        assert np.array_equal(ra["lse"], rb["lse"])


def test_mtp2_sequence_small():
    wl = get_workload("tiny-4k").with_(mtp=2, steps=3, ctx_len=2048,
                                      pool_slots=768, topk=128)
    recs = _run(wl)
    for r in recs[1:]:
        assert r["n_sel"].tolist() == [128, 128]
        wr = (r["row_dst"] >= 0).sum()
        assert wr == r["n_miss"]


def test_page_byte_arithmetic():
    g = load("page_numbers.txt")
    kap = footprint.kappa_base(g["l_kv"], g["d_kv"], g["l_index"], g["d_index"],
                               g["elem_bytes"])
    assert kap == 95232 and round(kap / 1000, 2) == g["kappa_kB"]
    kv = footprint.kv_part(g["l_kv"], g["d_kv"], g["elem_bytes"])
    ix = footprint.index_part(g["l_index"], g["d_index"], g["elem_bytes"])
    assert round(kv / 1000, 2) == g["kv_kB"] and round(ix / 1000, 2) == g["index_kB"]
    assert round(100 * ix / kap, 1) == g["index_share_pct"]
    for t, gb in ((g["tokens_64k"], g["gb_64k"]), (g["tokens_512k"], g["gb_512k"]),
                  (g["tokens_1m"], g["gb_1m"])):
        assert round(footprint.request_bytes(kap, t) / 1e9, 2) == gb
    assert round(100 * footprint.prefill_buffer_share(g["l_kv"]), 1) == g["prefill_share_pct"]
    r64 = footprint.decode_resident_bytes(kv, ix, g["hot_16k_tokens"], g["tokens_64k"])
    assert round(r64 / 1e9, 2) == g["resident_64k_gb"]
    # The page multiplies the rounded per-token figures (89.86 kB, 5.38 kB).
    hot = 89.86e3 * g["hot_128k_tokens"]
    idx = 5.38e3 * g["ctx_128k_tokens"]
    assert round(hot / 1e9, 2) == g["hot_128k_gb"]
    assert round(idx / 1e9, 2) == g["index_128k_gb"]
    assert round((hot + idx) / 1e9, 1) == g["per_req_128k_gb"]
    assert round(6 * (hot + idx) / 1e9) == g["six_req_128k_gb"]


def test_page_overlap_ratio():
    g = load("page_numbers.txt")
    r = footprint.overlap_ratio(g["t_copy_us"], g["t_sfa_us"], g["t_fused_us"])
    assert abs(r - g["overlap"]) < 1e-9
    speedup = (g["t_copy_us"] + g["t_sfa_us"]) / g["t_fused_us"]
    assert g["speedup_lo"] <= speedup <= g["speedup_hi"]
    # Fully hidden copy gives 1, fully exposed gives 0.
    assert footprint.overlap_ratio(10, 50, 50) == 1.0
    assert footprint.overlap_ratio(10, 50, 60) == 0.0


def _small_growth(steps=6):
    wl = get_workload("tiny-4k").with_(name="grow", mtp=2, ctx_len=600,
                                       topk=700, pool_slots=1400, steps=steps)
    return wl, 600 - 2 * steps - 3


def test_growth_dense_sees_each_new_token():
    # k above every visible length: step t token j selects exactly the
    # positions 0 .. L0 + 2t + j (its own included), so each appended
    # token is selected from the step that appends it; the pool holds every
    # position seen so far, and each step's misses are its two new tokens
    # (the fill covered token 0's view of the first L0 positions).
    wl, L0 = _small_growth()
    it = decode.run_workload_request(wl, 0, 0, grow_from=L0)
    fill = next(it)
    assert fill["n_miss"] == L0 - 1
    for t, rec in enumerate(it):
        for j in range(2):
            n = L0 + 2 * t + 1 + j
            assert rec["n_sel"][j] == n
            assert sorted(rec["sel_pos"][j, :n].tolist()) == list(range(n))
        # Step 0 also brings in L0 - 1, which the fill's token 0 did not see.
        expect = [L0 - 1, L0, L0 + 1] if t == 0 else [L0 + 2 * t, L0 + 2 * t + 1]
        assert rec["miss_pos"].tolist() == expect


def test_growth_with_fixed_lengths_is_the_static_run():
    # n_vis_fn returning the static lengths every step changes nothing.
    wl = get_workload("tiny-4k").with_(steps=3)
    a = list(decode.run_workload_request(wl, 0, 0))
    fixed = [wl.n_vis(j) for j in range(wl.mtp)]
    b = list(decode.run_workload_request(wl, 0, 0, n_vis_fn=lambda t: fixed))
    for ra, rb in zip(a[1:], b[1:]):
        for key in ("sel_pos", "n_sel", "miss_pos", "out", "lse"):
            assert np.array_equal(ra[key], rb[key]), key
