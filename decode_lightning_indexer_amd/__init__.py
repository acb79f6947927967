"""MI355X (gfx950) sparse decode over a host-offloaded latent cache.

The compute path is libess.so (HIP kernels behind the C ABI in
include/ess.h); `ess` is its ctypes binding and `session` holds buffer
plumbing over PyTorch device memory and the library's pinned host store.
"""
from . import ess  # noqa: F401
