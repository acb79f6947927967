"""Workload shapes for one decode step of DSA-style sparse attention over an
offloaded latent cache.

Each workload fixes the request count B, the query tokens per step m (MTP ways
sharing one pool), the cached positions L, the indexer geometry, top-k, the
MLA head count, the hot-pool slots C, the number of decode steps T, the layer
count and the AR(1) drift coefficient rho of the indexer queries.

Latent width 576 = c_KV[512] + k_R[64] and the 512-wide value part follow the
DSA latent layout described on the ESS concept page ("双 Cache 与 ESS 分工",
the table of what each cache stores).  The softmax scale 1/sqrt(576) = 1/24 is
the plain dot-product reading over the 576-wide key; the pages leave it open.
"""
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int          # B requests
    mtp: int            # m query tokens per step sharing one pool
    ctx_len: int        # L cached positions
    idx_heads: int      # H_I indexer heads
    idx_dim: int        # d_I indexer dim
    topk: int           # k
    mla_heads: int      # H absorbed-MLA query heads
    pool_slots: int     # C hot-pool slots per request (per layer)
    steps: int          # T decode steps
    layers: int         # N_L layers
    rho: float          # AR(1) coefficient of the indexer-query drift
    seed: int
    miss_mode: str      # "inline" (misses read inside attention) | "prefetch"
    lat_dim: int = 576
    v_dim: int = 512

    @property
    def softmax_scale(self) -> float:
        return 1.0 / 24.0

    def n_vis(self, j: int) -> int:
        """Visible positions of query token j: the m query tokens of a step are
        the last m positions, so token j sees L - m + 1 + j of them."""
        return self.ctx_len - self.mtp + 1 + j

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


_BASE = dict(idx_heads=64, idx_dim=128, topk=2048, mla_heads=128)

WORKLOADS = {
    # Oracle-sized single layer: 4K context, 8 steps.
    "tiny-4k": Workload("tiny-4k", batch=1, mtp=1, ctx_len=4096, idx_heads=16,
                        idx_dim=64, topk=256, mla_heads=16, pool_slots=1024,
                        steps=8, layers=1, rho=0.95, seed=0,
                        miss_mode="inline"),
    # V3.2-shaped single layer at 32K context.
    "32k-b16": Workload("32k-b16", batch=16, mtp=1, ctx_len=32768,
                        pool_slots=8192, steps=32, layers=1, rho=0.95, seed=1,
                        miss_mode="inline", **_BASE),
    # 128K context with two MTP ways sharing one pool; rho sweep.
    "128k-b8-mtp2-r099": Workload("128k-b8-mtp2-r099", batch=8, mtp=2,
                                  ctx_len=131072, pool_slots=16384, steps=32,
                                  layers=1, rho=0.99, seed=2,
                                  miss_mode="inline", **_BASE),
    "128k-b8-mtp2-r095": Workload("128k-b8-mtp2-r095", batch=8, mtp=2,
                                  ctx_len=131072, pool_slots=16384, steps=32,
                                  layers=1, rho=0.95, seed=2,
                                  miss_mode="inline", **_BASE),
    "128k-b8-mtp2-r080": Workload("128k-b8-mtp2-r080", batch=8, mtp=2,
                                  ctx_len=131072, pool_slots=16384, steps=32,
                                  layers=1, rho=0.80, seed=2,
                                  miss_mode="inline", **_BASE),
    # 16-layer loop at 64K with side-stream prefetch of the next layer.
    "64k-b32-16layer": Workload("64k-b32-16layer", batch=32, mtp=1,
                                ctx_len=65536, pool_slots=16384, steps=16,
                                layers=16, rho=0.95, seed=3,
                                miss_mode="prefetch", **_BASE),
    # 1M-token single request, hot-pool budget ablation.
    "1m-b1-c8k": Workload("1m-b1-c8k", batch=1, mtp=1, ctx_len=1 << 20,
                          idx_heads=32, idx_dim=128, topk=2048, mla_heads=64,
                          pool_slots=8192, steps=8, layers=1, rho=0.95, seed=4,
                          miss_mode="inline"),
    "1m-b1-c16k": Workload("1m-b1-c16k", batch=1, mtp=1, ctx_len=1 << 20,
                           idx_heads=32, idx_dim=128, topk=2048, mla_heads=64,
                           pool_slots=16384, steps=8, layers=1, rho=0.95,
                           seed=4, miss_mode="inline"),
}


def get_workload(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}")
