"""The four-buffer prefill pipeline on the GPU (ess_prefill_layers) against
the oracle: buffer bindings, per-layer column sums and the host store after
the write-backs, all bit-exact (integer-valued bf16 data)."""
import numpy as np
import pytest
import torch

from decode_lightning_indexer_amd import ess
from decode_lightning_indexer_amd.session import HostStore
from oracle import prefill as oprefill
from synth.gen import f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def _data(rng, NL, rows, n_new):
    host = f32_to_bf16_bits(rng.integers(-8, 9, (NL, rows, 576)).astype(np.float32))
    new = f32_to_bf16_bits(rng.integers(-8, 9, (NL, n_new, 576)).astype(np.float32))
    return host, new


@pytest.mark.parametrize("NL,rows,n_hist,n_new,onload,reps,load0", [
    (7, 3000, 2500, 300, None, 1, True),
    (7, 3000, 2500, 300, [-1, -1, 4, 5, 6, -1, -1], 3, True),   # loads one layer later
    (2, 700, 600, 77, None, 2, False),                           # B0 preloaded by hand
    (5, 1100, 0, 1029, None, 1, True),                           # no history: a first chunk
    (6, 2049, 2049, 0, None, 1, True),                           # nothing new: loads only
    (1, 64, 40, 24, None, 1, False),
])
def test_prefill_matches_oracle(NL, rows, n_hist, n_new, onload, reps, load0):
    rng = np.random.default_rng(NL * 100 + rows)
    host_np, new_np = _data(rng, NL, rows, n_new)
    store = HostStore((NL, rows, 576))
    store.array[:] = host_np
    dev = "cuda"
    new = torch.from_numpy(new_np.view(np.int16)).to(dev) if n_new else torch.empty(1, dtype=torch.int16, device=dev)
    bufs = torch.full((4, rows, 576), 0x7FC0, dtype=torch.int16, device=dev)   # NaN fill
    if not load0:
        bufs[0, :n_hist] = torch.from_numpy(host_np[0, :n_hist].view(np.int16)).to(dev)
    out = torch.zeros((NL, 576), dtype=torch.float32, device=dev)
    ws = torch.empty(ess.ess_prefill_ws_bytes(rows), dtype=torch.uint8, device=dev)
    s_c, s_h, s_d = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()            # inputs written on the default stream
    with torch.cuda.stream(s_c):
        binding = ess.ess_prefill_layers(
            NL, rows, n_hist, n_new, store.host, new, bufs, out, ws,
            onload_layer_map=onload, compute_reps=reps, load_layer0=load0,
            compute=s_c, h2d=s_h, d2h=s_d)
    s_c.synchronize()
    bind_ref, _, _ = oprefill.schedule(NL, onload)
    after_ref, out_ref = oprefill.run(host_np, new_np, n_hist)
    assert binding.tolist() == bind_ref
    assert np.array_equal(out.cpu().numpy().astype(np.float64), out_ref)
    assert np.array_equal(store.array, after_ref)
    store.free()


def test_prefill_rejects_a_map_that_leaves_a_layer_unloaded():
    NL, rows = 6, 64
    store = HostStore((NL, rows, 576))
    dev = "cuda"
    new = torch.zeros((NL, 8, 576), dtype=torch.int16, device=dev)
    bufs = torch.zeros((4, rows, 576), dtype=torch.int16, device=dev)
    out = torch.zeros((NL, 576), dtype=torch.float32, device=dev)
    ws = torch.empty(ess.ess_prefill_ws_bytes(rows), dtype=torch.uint8, device=dev)
    s = [torch.cuda.Stream() for _ in range(3)]
    with pytest.raises(ess.EssError) as e:
        ess.ess_prefill_layers(NL, rows, 32, 8, store.host, new, bufs, out, ws,
                               onload_layer_map=[-1] * NL, compute=s[0], h2d=s[1], d2h=s[2])
    assert e.value.status == "invalid argument"
    store.free()
