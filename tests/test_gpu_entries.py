"""656-byte fp8 latent entries on the GPU.

The dequantizing miss copy (ess_miss_copy_entries) against the oracle's
decoder, bit-exact; the attention reading misses as entries
(ess_sparse_mla_decode_entries) against the same attention over the
dequantized rows, bit-exact, and the oracle; whole decode sequences whose
host store holds entries: output for output equal to the bf16 path over the
dequantized latents, and within the attention tolerance of the oracle run on
those latents."""
import numpy as np
import pytest
import torch

from decode_lightning_indexer_amd import ess
from decode_lightning_indexer_amd.session import HostStore
from oracle.attention import attend
from oracle.formats import decode_entries
from synth import gen, get_workload
from tests.gpu_util import (assert_attn_close, compare_with_oracle, dequantized_latents,
                            dims, gpu_sequence, h, lse_close, sync, t)

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0     # fill of pool slots no copy may touch


def _expected_rows(entries):
    return gen.f32_to_bf16_bits(decode_entries(entries).astype(np.float32))


def _copy(entries, mp, ms, counts, C):
    B, L, _ = entries.shape
    stride = mp.shape[1]
    store = HostStore((B, L, 656), np.uint8)
    store.array[:] = entries
    d = dims(batch=B, ctx_len=L, pool_slots=C, topk=min(64, C))
    pool = torch.full((B, C, 576), NAN_BF16, dtype=torch.int16, device="cuda")
    print(f"entry copy B={B} L={L} C={C} stride={stride} counts={counts}", flush=True)
    ess.ess_miss_copy_entries(d, stride, t(mp), t(ms), t(np.int32(counts)), store.dev, pool)
    sync()
    got = h(pool)
    store.free()
    exp = np.full((B, C, 576), NAN_BF16, np.uint16)
    for b, n in enumerate(counts):
        n = min(n, stride)
        ok = (mp[b, :n] >= 0) & (ms[b, :n] >= 0)
        exp[b, ms[b, :n][ok]] = _expected_rows(entries[b, mp[b, :n][ok]])
    return got, exp


@pytest.mark.parametrize("B,L,C,stride,counts", [
    (1, 100, 64, 64, [37]),
    (3, 5000, 3000, 2048, [2048, 0, 777]),     # a full list, an empty one, a ragged one
    (2, 300, 300, 300, [300, 299]),            # every slot written
    (2, 4000, 1024, 512, [1000, 23]),          # count beyond the list: the list caps it
])
def test_entry_copy_matches_decoder(B, L, C, stride, counts):
    rng = np.random.default_rng(B * 1000 + L)
    mag = rng.choice([1e-3, 0.5, 40.0], (B, L, 1))              # rows of very different ranges
    lat = gen.f32_to_bf16_bits((rng.standard_normal((B, L, 576)) * mag).astype(np.float32))
    ent = gen.encode_entries(lat.reshape(-1, 576)).reshape(B, L, 656)
    mp = np.full((B, stride), -1, np.int32)
    ms = np.full((B, stride), -1, np.int32)
    for b, n in enumerate(counts):
        n = min(n, stride)
        mp[b, :n] = rng.choice(L, n, replace=False)
        ms[b, :n] = rng.choice(C, n, replace=False)
    if counts[0] > 4:
        mp[0, 3] = -1                      # an entry outside the store: skipped
    got, exp = _copy(ent, mp, ms, counts, C)
    assert np.array_equal(got, exp)


def test_entry_copy_every_code_and_scale():
    # Hand-built entries: c_KV runs through every e4m3fn code but the two
    # NaNs (0x80 is -0), scales from 2^-20 to 2^20, arbitrary k_R bits.
    B, L, C = 2, 16, 16
    rng = np.random.default_rng(5)
    ent = np.zeros((B, L, 656), np.uint8)
    for b in range(B):
        for s in range(L):
            q = (np.arange(512) + 37 * s + b) % 256
            q[q == 0x7F] = 0x7E
            q[q == 0xFF] = 0xFE
            ent[b, s, :512] = q
            sc = 2.0 ** (np.arange(4) + (s % 10) * 4 - 20)
            ent[b, s, 512:528] = sc.astype(np.float32).view(np.uint8)
            kr = gen.f32_to_bf16_bits(rng.standard_normal(64).astype(np.float32) * 3)
            ent[b, s, 528:] = kr.view(np.uint8)
    mp = np.tile(np.arange(L, dtype=np.int32), (B, 1))
    ms = np.stack([rng.permutation(C).astype(np.int32) for _ in range(B)])
    got, exp = _copy(ent, mp, ms, [L, L], C)
    assert np.array_equal(got, exp)


def _wl():
    return get_workload("tiny-4k").with_(name="entries", batch=2, steps=4)


@pytest.mark.parametrize("mode", [ess.ESS_MODE_INLINE, ess.ESS_MODE_PREFETCH])
def test_entry_store_equals_bf16_path_on_dequantized_latents(mode):
    wl = _wl().with_(layers=2)
    a = gpu_sequence(wl, mode=mode, store="entries")
    b = gpu_sequence(wl, mode=mode, store="dequantized")
    assert sum(int(s[0]["n_miss"].sum()) for s in a["steps"]) > 0
    for fa, fb in zip(a["fill"], b["fill"]):
        for key in fa:
            assert np.array_equal(fa[key], fb[key]), key
    for sa, sb in zip(a["steps"], b["steps"]):
        for la, lb in zip(sa, sb):
            for key in la:
                assert np.array_equal(la[key], lb[key]), key


def test_entry_store_matches_oracle():
    wl = _wl().with_(name="entries-mtp2", mtp=2, pool_slots=2048, topk=512,
                     steps=5, rho=0.9)
    recs = gpu_sequence(wl, store="entries")
    _, eff = dequantized_latents(wl, 0)
    compare_with_oracle(wl, recs, host=eff)


def _selection(rng, B, m, L, k, C, ragged, p_hit):
    """Selected rows per (request, token), hits with their slots, misses with
    one designated writer each, and writer slots planted past n_sel."""
    n_sel = np.zeros((B, m), np.int32)
    sel = np.full((B, m, k), -1, np.int32)
    src = np.full((B, m, k), -1, np.int32)
    dst = np.full((B, m, k), -1, np.int32)
    hit_rows = []
    for b in range(B):
        slot_of, free = {}, list(rng.permutation(C))
        for j in range(m):
            n = int(rng.integers(1, min(k, L) + 1)) if ragged else min(k, L)
            n_sel[b, j] = n
            pos = rng.permutation(L)[:n]
            sel[b, j, :n] = pos
            for i, p in enumerate(pos.tolist()):
                if p not in slot_of:
                    s, hit = free.pop(), rng.random() < p_hit
                    slot_of[p] = (s, hit)
                    if hit:
                        hit_rows.append((b, s, p))
                    else:
                        dst[b, j, i] = s
                s, hit = slot_of[p]
                src[b, j, i] = s if hit else -1
        for j in range(m):
            for i in range(n_sel[b, j], min(n_sel[b, j] + 2, k)):
                if free:
                    sel[b, j, i] = i % L
                    dst[b, j, i] = free.pop()
    return n_sel, sel, src, dst, hit_rows


@pytest.mark.parametrize("B,m,H,L,k,C,ragged,p_hit", [
    (1, 1, 16, 4096, 256, 1024, False, 0.8),
    (2, 2, 128, 2000, 512, 1200, True, 0.7),
    (1, 1, 32, 500, 45, 100, False, 0.0),      # all misses
    (1, 1, 48, 500, 33, 100, False, 1.0),      # all hits
    (8, 2, 128, 6000, 2048, 4200, True, 0.5),  # 8 chunks of 256 rows per token
])
def test_attention_over_entries_equals_bf16_rows(B, m, H, L, k, C, ragged, p_hit):
    # The attention reading misses as fp8 entries gives, bit for bit, what it
    # gives reading the dequantized rows as bf16, writes the same rows to the
    # slots, and is within the attention tolerance of the oracle.
    rng = np.random.default_rng(H * 11 + k)
    lat = gen.f32_to_bf16_bits((rng.standard_normal((B, L, 576)) * 0.5).astype(np.float32))
    ent_np = gen.encode_entries(lat.reshape(-1, 576)).reshape(B, L, 656)
    eff = _expected_rows(ent_np.reshape(-1, 656)).reshape(B, L, 576)
    ents = HostStore((B, L, 656), np.uint8)
    ents.array[:] = ent_np
    rows = HostStore((B, L, 576))
    rows.array[:] = eff
    qa = gen.f32_to_bf16_bits((rng.standard_normal((B, m, H, 576)) * 0.1).astype(np.float32))
    n_sel, sel, src, dst, hit_rows = _selection(rng, B, m, L, k, C, ragged, p_hit)
    pool = np.zeros((B, C, 576), np.uint16)
    for b, s, p in hit_rows:
        pool[b, s] = eff[b, p]
    d = dims(batch=B, mtp=m, ctx_len=L, mla_heads=H, topk=k, pool_slots=C)
    ws_bytes = ess.ess_workspace_bytes(d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    res = []
    for mode in ("entries", "bf16"):
        print(f"attention over {mode}: B={B} m={m} H={H} L={L} k={k} C={C}", flush=True)
        pool_t = t(pool)
        out = torch.empty((B, m, H, 512), dtype=torch.float32, device="cuda")
        lse = torch.empty((B, m, H), dtype=torch.float32, device="cuda")
        args = (d, t(qa), t(sel), t(src), t(dst), t(n_sel), pool_t)
        if mode == "entries":
            ess.ess_sparse_mla_decode_entries(*args, ents.dev, out, lse, ws, ws_bytes)
        else:
            ess.ess_sparse_mla_decode(*args, rows.dev, out, lse, ws, ws_bytes)
        sync()
        res.append((h(out), h(lse), h(pool_t)))
    (o1, l1, p1), (o2, l2, p2) = res
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert np.array_equal(p1, p2)
    for b in range(B):
        for j in range(m):
            n = n_sel[b, j]
            ref, rlse = attend(qa[b, j], eff[b, sel[b, j, :n]], 1 / 24)
            assert_attn_close(o1[b, j], ref, (b, j))
            lse_close(l1[b, j], rlse, (b, j))
        for j in range(m):
            for i in np.nonzero(dst[b, j, :n_sel[b, j]] >= 0)[0]:
                assert np.array_equal(p1[b, dst[b, j, i]], eff[b, sel[b, j, i]])
    ents.free()
    rows.free()
