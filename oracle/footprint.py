"""The pages' byte arithmetic for the offloaded cache.

FlashOffloading analysis, section "how 95.23 kB per token comes about":
the resident cost per token is the KV part plus the indexer state,
kappa_base = (L_KV * D_KV + L_index * D_index) * P bytes, and a request of
length T costs kappa_base * T.  The page's units are decimal (kB = 1000 B,
GB = 1e9 B) and its "64k", "512k", "1M" token counts are 64,000, 512,000
and 1,024,000 (the only reading that reproduces its 6.09, 48.76 and
97.52 GB).

Same page, section "4/L and (C+2b)/T": decode keeps per layer C hot tokens
plus two tail blocks of b tokens, M_decode ~ L (C + 2b) s_KV + M_index + ...,
and prefill keeps four full-layer buffers, a 4/L share.

Same page, section "numbers: 1.03x to 1.27x": OverlapRatio =
(T_copy + T_SFA - T_fused) / T_copy.
"""


def kappa_base(l_kv, d_kv, l_index, d_index, elem_bytes):
    """Resident bytes per token: KV part plus indexer state."""
    return (l_kv * d_kv + l_index * d_index) * elem_bytes


def kv_part(l_kv, d_kv, elem_bytes):
    return l_kv * d_kv * elem_bytes


def index_part(l_index, d_index, elem_bytes):
    return l_index * d_index * elem_bytes


def request_bytes(kappa, tokens):
    return kappa * tokens


def decode_resident_bytes(kv_per_token, index_per_token, hot_tokens, ctx_tokens):
    """Per-request decode residency: the hot cache holds the KV part of
    hot_tokens positions; the indexer state of all ctx_tokens stays."""
    return kv_per_token * hot_tokens + index_per_token * ctx_tokens


def prefill_buffer_share(layers, buffers=4):
    return buffers / layers


def overlap_ratio(t_copy, t_attn, t_fused):
    """Share of the copy time hidden by the fused kernel."""
    return (t_copy + t_attn - t_fused) / t_copy
