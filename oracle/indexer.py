"""Lightning-indexer scoring.

The pages say the indexer cache stays resident on the GPU and that every
decode step the indexer scores all L cached positions and keeps the top 2048
(ESS concept page, "dual cache" table; FlashOffloading analysis, section on
cache_slots).  They do not print the score formula.  The reading taken is the
DSA lightning-indexer score with no scale and no bias:

    score[j][s] = sum_h w[j][h] * max(0, sum_d q[j][h][d] * k[s][d])

for query token j and positions s < n_vis[j]; positions at or beyond n_vis[j]
are not candidates and get -inf.

With integer q, k in [-7, 7] and integer w in [1, 4], every partial sum is an
integer of magnitude at most H_I * 4 * d_I * 49 (1,605,632 for 64 heads of
dim 128), so float64 here, float32 anywhere, and int64 all give the same
exact value in any summation order.
"""
import numpy as np

from .formats import decode_e4m3fn


def index_scores(q_bytes, w, k_bytes, n_vis):
    """Scores of one request.

    q_bytes: uint8 [m][H_I][d_I] fp8 e4m3fn index queries
    w:       float [m][H_I] head weights
    k_bytes: uint8 [L][d_I] fp8 e4m3fn index keys
    n_vis:   int [m] visible positions per query token
    returns  float64 [m][L]; -inf at s >= n_vis[j]
    """
    q = decode_e4m3fn(q_bytes)
    K = decode_e4m3fn(k_bytes)
    w = np.asarray(w, dtype=np.float64)
    m, L = q.shape[0], K.shape[0]
    out = np.full((m, L), -np.inf)
    for j in range(m):
        n = int(n_vis[j])
        logits = q[j] @ K[:n].T                 # [H_I, n] per-head dot products
        out[j, :n] = w[j] @ np.maximum(logits, 0.0)
    return out
