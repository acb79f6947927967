"""Absorbed-MLA attention over the selected latents.

The pages describe the main attention as reading only the top-k latent
entries, each c_KV[512] plus k^R, up-projecting with W^UK / W^UV and running
the core MLA (ESS concept page, "dual cache" table), and insist that offload
changes only where data sits, not the attention set or the result
(FlashOffloading analysis, opening and section "cache_slots").  With W^UK
absorbed into the query, the core is single-latent-head attention:

    z_i   = scale * <qa[h], lat_i[0:576]>
    p     = softmax_i(z)
    out_h = sum_i p_i * lat_i[0:512]          (before W^UV)
    lse_h = log sum_i exp(z_i)

The oracle is that definition in float64 over the selected rows.
"""
import numpy as np

from .formats import decode_bf16


def attend(qa_bits, rows_bits, scale: float, v_dim: int = 512):
    """qa_bits uint16 [H][D]; rows_bits uint16 [n][D] (n >= 1).

    returns out float64 [H][v_dim], lse float64 [H].
    """
    q = decode_bf16(qa_bits)
    X = decode_bf16(rows_bits)
    z = scale * (q @ X.T)                          # [H, n]
    zmax = z.max(axis=1, keepdims=True)
    e = np.exp(z - zmax)
    den = e.sum(axis=1, keepdims=True)
    out = (e @ X[:, :v_dim]) / den
    lse = zmax[:, 0] + np.log(den[:, 0])
    return out, lse
