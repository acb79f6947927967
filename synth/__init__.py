"""Seeded synthetic inputs for the sparse-decode path.

This package is shared by the CPU oracle's tests, the GPU parity tests and
the benchmark.  It holds no arithmetic of the method itself: it only draws
random tensors with the shapes and value distributions of the workloads and
encodes them into the storage formats the path consumes (fp8 e4m3fn bytes for
the indexer, bf16 bit patterns for the latents and absorbed queries).
"""
from .workloads import Workload, WORKLOADS, get_workload  # noqa: F401
from . import gen  # noqa: F401
