"""Uploads of the seeded synthetic inputs into the device buffers and the
pinned host store of the decode path (input plumbing for the GPU tests and
the benchmark; no arithmetic of the method)."""
import numpy as np
import torch

from . import gen


class LayerInputs:
    """Seeded inputs of one layer, drawn once and uploaded per step."""

    def __init__(self, wl, layer):
        self.wl = wl
        self.layer = layer
        self.q, self.w, self.n_vis = gen.index_inputs(wl, layer)

    def upload_static(self, bufs, host_array, keys=True, latents=True):
        """Index keys to device, head weights, latents into the host store."""
        wl = self.wl
        if keys:
            kb = np.empty((wl.batch, wl.ctx_len, wl.idx_dim), np.uint8)
            gen.fill_index_keys(wl, self.layer, kb)
            bufs.k_idx.copy_(torch.from_numpy(kb))
            del kb
        bufs.w_idx.copy_(torch.from_numpy(self.w))
        if latents:
            gen.fill_latents(wl, self.layer, host_array)

    def upload_step(self, bufs, t):
        bufs.q_idx.copy_(torch.from_numpy(self.q[t]))
        qa = gen.abs_query(self.wl, self.layer, t)
        bufs.q_abs.copy_(torch.from_numpy(qa.view(np.int16)))

    def n_vis_tensor(self, device="cuda"):
        return torch.from_numpy(self.n_vis).to(device)
