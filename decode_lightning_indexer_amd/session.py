"""Buffers for running the decode path through the C ABI.

PyTorch provides device memory and streams; the latent store lives in pinned
host memory allocated by the library (ess_host_alloc) and is exposed here as
a NumPy array over the host address, so it can be filled in place.  Nothing
here computes any step of the path.
"""
import ctypes
import weakref

import numpy as np
import torch

from . import ess


class HostStore:
    """Pinned, device-mapped host array (bf16 bits as uint16 by default)."""

    def __init__(self, shape, dtype=np.uint16):
        self.shape = tuple(int(s) for s in shape)
        self.dtype = np.dtype(dtype)
        self.nbytes = int(np.prod(self.shape)) * self.dtype.itemsize
        self.host, self.dev = ess.ess_host_alloc(self.nbytes)
        buf = (ctypes.c_uint8 * self.nbytes).from_address(self.host)
        self.array = np.frombuffer(buf, dtype=self.dtype).reshape(self.shape)
        # Freed by free(), when the object is collected, or at the latest by
        # the interpreter's exit handlers, before the HIP runtime is torn down.
        self._fin = weakref.finalize(self, ess.ess_host_free, self.host)

    def free(self):
        if self.host:
            self.array = None
            self._fin()
            self.host = self.dev = 0


def dims_of(wl, **over) -> ess.ess_dims:
    kw = dict(batch=wl.batch, mtp=wl.mtp, ctx_len=wl.ctx_len,
              idx_heads=wl.idx_heads, idx_dim=wl.idx_dim,
              mla_heads=wl.mla_heads, topk=wl.topk,
              pool_slots=wl.pool_slots, softmax_scale=wl.softmax_scale)
    kw.update(over)
    return ess.make_dims(**kw)


class LayerBuffers:
    """Device buffers of one layer; `io()` packs them for ess_decode_step."""

    def __init__(self, d: ess.ess_dims, host: HostStore, device="cuda",
                 entries: HostStore = None):
        B, m, L = d.batch, d.mtp, d.ctx_len
        C, k, H = d.pool_slots, d.topk, d.mla_heads
        lists = max(m * k, C)
        i32 = dict(dtype=torch.int32, device=device)
        self.d = d
        self.host = host            # bf16 rows [B][L][576] (or None)
        self.entries = entries      # 656-byte fp8 entries [B][L][656] (or None)
        self.k_idx = torch.empty((B, L, d.idx_dim), dtype=torch.uint8, device=device)
        self.q_idx = torch.empty((B, m, d.idx_heads, d.idx_dim), dtype=torch.uint8,
                                 device=device)
        self.w_idx = torch.empty((B, m, d.idx_heads), dtype=torch.float32, device=device)
        self.q_abs = torch.empty((B, m, H, 576), dtype=torch.int16, device=device)
        self.pool = torch.zeros((B, C, 576), dtype=torch.int16, device=device)
        self.cache_slots = torch.empty((B, L), **i32)
        self.slot_pos = torch.empty((B, C), **i32)
        self.lru = torch.empty(ess.ess_lru_state_bytes(d), dtype=torch.uint8,
                               device=device)
        self.scores = torch.empty((B, m, L), dtype=torch.float32, device=device)
        self.sel_pos = torch.empty(B * lists, **i32)
        self.sel_slot = torch.empty(B * lists, **i32)
        self.row_dst = torch.empty(B * lists, **i32)
        self.sel_slot_post = torch.empty(B * lists, **i32)
        self.n_sel = torch.empty((B, m), **i32)
        self.miss_pos = torch.empty(B * lists, **i32)
        self.miss_slot = torch.empty(B * lists, **i32)
        self.n_miss = torch.empty(B, **i32)
        self.n_evict = torch.empty(B, **i32)
        self.out = torch.empty((B, m, H, 512), dtype=torch.float32, device=device)
        self.lse = torch.empty((B, m, H), dtype=torch.float32, device=device)
        self.ws_bytes = ess.ess_workspace_bytes(d)
        self.ws = torch.empty(max(1, self.ws_bytes), dtype=torch.uint8, device=device)

    def reset(self, stream=None):
        ess.ess_pool_reset(self.d, self.cache_slots, self.slot_pos, self.lru,
                           stream)

    def io(self) -> ess.ess_layer_io:
        p = lambda t: t.data_ptr()
        return ess.ess_layer_io(
            p(self.q_idx), p(self.w_idx), p(self.k_idx), p(self.q_abs),
            self.host.dev if self.host else None, p(self.pool),
            p(self.cache_slots), p(self.slot_pos),
            p(self.lru), p(self.scores), p(self.sel_pos), p(self.sel_slot),
            p(self.n_sel), p(self.row_dst), p(self.sel_slot_post),
            p(self.miss_pos), p(self.miss_slot), p(self.n_miss),
            p(self.n_evict), p(self.out), p(self.lse), p(self.ws),
            self.ws_bytes, self.entries.dev if self.entries else None)

    def rows(self, t, k, n_tok):
        """View of a flat per-row array as [B][n_tok][k]."""
        B = self.d.batch
        return t[:B * n_tok * k].view(B, n_tok, k)

    def lists(self, t, stride):
        B = self.d.batch
        return t[:B * stride].view(B, stride)
