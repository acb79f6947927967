"""Pins for the oracle's attention: a second route through PyTorch's CPU
scaled_dot_product_attention in float64 with a boolean mask over all
positions, the dense (k >= L) case, and closed forms."""
import numpy as np
import torch

from oracle.attention import attend
from oracle.formats import decode_bf16
from oracle.topk import topk_positions
from synth import gen


def _sdpa_masked(qa_bits, host_bits, mask, scale, v_dim=512):
    q = torch.from_numpy(decode_bf16(qa_bits))[None]          # [1, H, D]
    X = torch.from_numpy(decode_bf16(host_bits))               # [L, D]
    k = X[None, None].expand(1, q.shape[1], -1, -1)            # [1, H, L, D]
    v = X[None, None, :, :v_dim].expand(1, q.shape[1], -1, -1)
    m = torch.from_numpy(mask)[None, None, None, :].expand(1, q.shape[1], 1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(
        q[:, :, None, :], k, v, attn_mask=m, scale=scale)
    return o[0, :, 0, :].numpy()


def test_attention_matches_masked_sdpa_over_topk_set():
    rng = np.random.default_rng(4)
    L, H, D, k = 300, 8, 576, 40
    host = gen.f32_to_bf16_bits(rng.standard_normal((L, D)).astype(np.float32) * 0.5)
    qa = gen.f32_to_bf16_bits(rng.standard_normal((H, D)).astype(np.float32) * 0.1)
    scores = rng.integers(0, 50, L).astype(np.float64)
    sel = topk_positions(scores, L, k)
    out, lse = attend(qa, host[sel], 1 / 24)
    mask = np.zeros(L, bool)
    mask[sel] = True
    ref = _sdpa_masked(qa, host, mask, 1 / 24)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)
    # lse by direct summation in another order.
    z = (decode_bf16(qa) @ decode_bf16(host[np.sort(sel)]).T) / 24
    np.testing.assert_allclose(lse, np.log(np.exp(z).sum(1)), rtol=1e-12)


def test_k_at_least_L_is_dense_mla():
    rng = np.random.default_rng(6)
    L, H, D = 50, 4, 576
    host = gen.f32_to_bf16_bits(rng.standard_normal((L, D)).astype(np.float32) * 0.5)
    qa = gen.f32_to_bf16_bits(rng.standard_normal((H, D)).astype(np.float32))
    sel = topk_positions(rng.standard_normal(L), L, 10 * L)
    assert sorted(sel.tolist()) == list(range(L))
    out, _ = attend(qa, host[sel], 0.3)
    ref = _sdpa_masked(qa, host, np.ones(L, bool), 0.3)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def test_closed_forms():
    D = 576
    row = gen.f32_to_bf16_bits(np.linspace(-1, 1, D).astype(np.float32))
    qa = gen.f32_to_bf16_bits(np.full((3, D), 0.01, np.float32))
    # One row: softmax weight 1, out = the row's value part, lse = z.
    out, lse = attend(qa, row[None], 0.5)
    v = decode_bf16(row)
    np.testing.assert_array_equal(out, np.broadcast_to(v[:512], (3, 512)))
    z = 0.5 * decode_bf16(qa) @ v
    np.testing.assert_allclose(lse, z, rtol=1e-14)
    # n identical rows: same out, lse = z + log n.
    out, lse = attend(qa, np.repeat(row[None], 7, 0), 0.5)
    np.testing.assert_allclose(out, np.broadcast_to(v[:512], (3, 512)), rtol=1e-14)
    np.testing.assert_allclose(lse, z + np.log(7), rtol=1e-14)


def test_only_the_first_512_columns_are_values():
    D = 576
    rng = np.random.default_rng(1)
    rows = gen.f32_to_bf16_bits(rng.standard_normal((5, D)).astype(np.float32))
    rows2 = rows.copy()
    qa = np.zeros((2, D), np.uint16)           # zero query: uniform weights
    out, _ = attend(qa, rows, 1.0)
    rows2[:, 512:] = 0
    out2, _ = attend(qa, rows2, 1.0)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_allclose(out[0], decode_bf16(rows)[:, :512].mean(0), rtol=1e-12)
