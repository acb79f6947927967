"""The library's eviction-policy replay (a host routine, ess_replay_evictions)
against the oracle's replay: miss and eviction counts equal step by step."""
import numpy as np
import pytest

from decode_lightning_indexer_amd import ess
from oracle.policies import replay
from tests.test_oracle_policies import _random_scores, _sel

CODES = {"lru": ess.ESS_EVICT_LRU, "random": ess.ESS_EVICT_RANDOM,
         "score": ess.ESS_EVICT_SCORE}


@pytest.fixture(scope="module")
def L():
    return ess.lib()


@pytest.mark.parametrize("policy", sorted(CODES))
@pytest.mark.parametrize("T,m,Lc,k,C,drift,ragged", [
    (12, 1, 800, 50, 120, 0.9, False),
    (10, 2, 1500, 64, 256, 0.8, True),
    (8, 3, 600, 30, 90, 0.95, False),      # union of three ways fills C
    (15, 2, 400, 40, 2000, 0.7, False),    # C > L: no evictions
    (6, 1, 300, 100, 100, 0.5, True),      # C = k: every miss evicts
])
def test_replay_matches_the_oracle(L, policy, T, m, Lc, k, C, drift, ragged):
    rng = np.random.default_rng(T * 1000 + Lc + m)
    s = _random_scores(rng, T, m, Lc, drift=drift).astype(np.float32)
    if ragged:
        for j in range(m):
            s[:, j, Lc - 1 - j * 13:] = -np.inf
    sel, n = _sel(s.astype(np.float64), k)
    for req, seed in ((0, 0), (5, 0xDEADBEEF)):
        got_m, got_e = ess.ess_replay_evictions(CODES[policy], C, s, sel, n,
                                                seed=seed, request=req)
        ref_m, ref_e = replay(s, sel, n, C, policy, seed=seed, request=req)
        assert np.array_equal(got_m, ref_m) and np.array_equal(got_e, ref_e), (req, seed)


def test_replay_errors(L):
    rng = np.random.default_rng(0)
    s = _random_scores(rng, 3, 2, 200).astype(np.float32)
    sel, n = _sel(s.astype(np.float64), 30)
    with pytest.raises(ess.EssError) as e:
        ess.ess_replay_evictions(ess.ESS_EVICT_LRU, 40, s, sel, n)    # two ways of 30 > 40
    assert e.value.status == "pool capacity exceeded"
    bad = sel.copy()
    bad[1, 0, 3] = 200
    with pytest.raises(ess.EssError) as e:
        ess.ess_replay_evictions(ess.ESS_EVICT_LRU, 100, s, bad, n)
    assert e.value.status == "invalid argument"
    with pytest.raises(ess.EssError):
        ess.ess_replay_evictions(7, 100, s, sel, n)
    with pytest.raises(ess.EssError):
        ess.ess_replay_evictions(ess.ESS_EVICT_LRU, 100, s, sel, n, request=1 << 16)
