"""Helpers shared by the GPU parity tests."""
import numpy as np
import torch

from decode_lightning_indexer_amd import ess

DEV = "cuda"

# Attention tolerance: max |d| <= 1e-2 * max |ref| and sum |d| / sum |ref|
# <= 2e-3 over all outputs of a step.
MAX_ABS_REL = 1e-2
MEAN_REL = 2e-3


def attn_errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = np.abs(got - ref)
    return d.max() / np.abs(ref).max(), d.sum() / np.abs(ref).sum()


def assert_attn_close(got, ref, what=""):
    mx, mean = attn_errors(got, ref)
    assert mx <= MAX_ABS_REL and mean <= MEAN_REL, (what, mx, mean)
    return mx, mean


def lse_close(got, ref, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.abs(got - ref).max() <= 1e-3 * max(1.0, np.abs(ref).max()), what


def t(x, dtype=None):
    """numpy -> device tensor (uint16 arrays travel as int16)."""
    a = np.ascontiguousarray(x)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    tt = torch.from_numpy(a)
    if dtype is not None:
        tt = tt.to(dtype)
    return tt.to(DEV)


def h(x):
    """device tensor -> numpy (int16 -> uint16 bits)."""
    a = x.detach().cpu().numpy()
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    return a


def sync():
    torch.cuda.synchronize()


def dims(**kw):
    base = dict(batch=1, mtp=1, ctx_len=1024, idx_heads=16, idx_dim=64,
                mla_heads=16, topk=64, pool_slots=256, softmax_scale=1 / 24)
    base.update(kw)
    return ess.make_dims(**base)
