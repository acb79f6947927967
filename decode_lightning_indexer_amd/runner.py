"""Drive whole decode steps over several layers through ess_decode_step.

Holds one LayerBuffers per layer, the shared n_vis tensor and the streams
(the caller's current stream, plus a second stream at default priority for
the prefetch mode).  Plumbing only: each step is one ess_decode_step call.
"""
import torch

from . import ess
from .session import LayerBuffers


class DecodeRunner:
    def __init__(self, d: ess.ess_dims, hosts, device="cuda", entries=None):
        """hosts: one bf16 HostStore per layer; entries: optionally one
        656-byte-entry HostStore per layer (the host store then holds fp8
        entries and hosts may hold None)."""
        self.d = d
        entries = entries if entries is not None else [None] * len(hosts)
        self.layers = [LayerBuffers(d, h, device, e) for h, e in zip(hosts, entries)]
        self.n_vis = torch.empty((d.batch, d.mtp), dtype=torch.int32,
                                 device=device)
        self.side = torch.cuda.Stream(device=device)
        self._ios = [lb.io() for lb in self.layers]

    def set_n_vis(self, n_vis):
        self.n_vis.copy_(torch.as_tensor(n_vis, dtype=torch.int32))

    def reset(self):
        for lb in self.layers:
            lb.reset()

    def fill(self, stream=None):
        ess.ess_decode_step(self.d, self._ios, self.n_vis, ess.ESS_MODE_FILL,
                            stream)

    def step(self, mode=ess.ESS_MODE_INLINE, stream=None):
        ess.ess_decode_step(self.d, self._ios, self.n_vis, mode, stream,
                            self.side)
