"""Pins for the oracle's indexer scores: brute force in integers, closed
forms, the ReLU, masking and the exactness bound."""
import numpy as np

from oracle.indexer import index_scores
from synth import gen


def _brute(qi, w, ki, n_vis):
    m, H, d = qi.shape
    L = ki.shape[0]
    out = [[None] * L for _ in range(m)]
    for j in range(m):
        for s in range(L):
            if s >= n_vis[j]:
                out[j][s] = float("-inf")
                continue
            tot = 0
            for h in range(H):
                dot = 0
                for e in range(d):
                    dot += int(qi[j, h, e]) * int(ki[s, e])
                tot += int(w[j, h]) * max(0, dot)
            out[j][s] = tot
    return out


def test_scores_match_integer_brute_force():
    rng = np.random.default_rng(11)
    m, H, d, L = 2, 4, 8, 37
    qi = rng.integers(-7, 8, (m, H, d))
    ki = rng.integers(-7, 8, (L, d))
    w = rng.integers(1, 5, (m, H)).astype(np.float32)
    n_vis = np.array([L - 1, L])
    got = index_scores(gen.encode_e4m3_int(qi), w, gen.encode_e4m3_int(ki), n_vis)
    ref = _brute(qi, w, ki, n_vis)
    assert np.array_equal(got, np.array(ref, dtype=np.float64))


def test_closed_forms():
    d, H, L = 64, 16, 10
    ones_q = gen.encode_e4m3_int(np.ones((1, H, d), np.int64))
    w = np.arange(1, H + 1, dtype=np.float32)[None, :] % 4 + 1
    # All +1 keys: every head's dot is d, the score is d * sum(w).
    k_pos = gen.encode_e4m3_int(np.ones((L, d), np.int64))
    s = index_scores(ones_q, w, k_pos, [L])
    assert np.all(s == d * w.sum())
    # All -1 keys: every dot is -d, ReLU zeroes it.
    k_neg = gen.encode_e4m3_int(-np.ones((L, d), np.int64))
    assert np.all(index_scores(ones_q, w, k_neg, [L]) == 0.0)
    # Extreme values: 7 * 7 * d per head.
    q7 = gen.encode_e4m3_int(np.full((1, H, d), 7))
    k7 = gen.encode_e4m3_int(np.full((L, d), -7))
    assert np.all(index_scores(q7, w, gen.encode_e4m3_int(np.full((L, d), 7)), [L])
                  == 49 * d * w.sum())
    assert np.all(index_scores(q7, w, k7, [L]) == 0.0)


def test_relu_is_per_head_before_weighting():
    # Head 0 dot = +d, head 1 dot = -d: only head 0 counts.
    d = 32
    q = np.zeros((1, 2, d), np.int64)
    q[0, 0] = 1
    q[0, 1] = -1
    k = np.ones((3, d), np.int64)
    w = np.array([[2.0, 3.0]], np.float32)
    s = index_scores(gen.encode_e4m3_int(q), w, gen.encode_e4m3_int(k), [3])
    assert np.all(s == 2.0 * d)


def test_masking_beyond_n_vis():
    rng = np.random.default_rng(3)
    q = gen.encode_e4m3_int(rng.integers(-7, 8, (2, 4, 32)))
    k = gen.encode_e4m3_int(rng.integers(-7, 8, (20, 32)))
    w = np.ones((2, 4), np.float32)
    s = index_scores(q, w, k, [5, 20])
    assert np.all(np.isneginf(s[0, 5:])) and np.all(np.isfinite(s[0, :5]))
    assert np.all(np.isfinite(s[1]))


def test_float32_exactness_bound_at_full_head_shape():
    # 64 heads x 128 dims with weights up to 4: the largest possible score
    # is below 2^24, so float32 accumulation reproduces the integers.
    assert 64 * 4 * 128 * 49 < 2 ** 24
    rng = np.random.default_rng(5)
    qi = rng.integers(-7, 8, (1, 64, 128))
    ki = rng.integers(-7, 8, (300, 128))
    w = rng.integers(1, 5, (1, 64)).astype(np.float32)
    s64 = index_scores(gen.encode_e4m3_int(qi), w, gen.encode_e4m3_int(ki), [300])
    dots = (qi[0].astype(np.float32) @ ki.T.astype(np.float32))
    s32 = (w[0] @ np.maximum(dots, 0)).astype(np.float32)
    si = (w[0].astype(np.int64) @ np.maximum(qi[0] @ ki.T, 0))
    assert np.array_equal(s64[0], si.astype(np.float64))
    assert np.array_equal(s32.astype(np.float64), s64[0])
