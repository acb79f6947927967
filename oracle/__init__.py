"""CPU oracle for one decode step of DSA-style sparse attention over a latent
cache offloaded to host memory.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this package.  The product path (the
HIP library and its Python binding) never imports, calls or links anything
here, and nothing here imports the product path.

Plain, slow and written to be checked by eye against the pages:
  * formats   - fp8 e4m3fn and bf16 decoding from the format definitions;
  * indexer   - lightning-indexer scores in float64;
  * topk      - full sort on (score descending, position ascending);
  * pool      - hot pool with an OrderedDict LRU, cache_slots reverse index
                and the five-step miss handling;
  * attention - dense float64 softmax over the selected latents;
  * decode    - a whole decode sequence (fill, then T steps) per request;
  * footprint - the pages' per-token byte arithmetic;
  * policies  - offline replay of the pool under the LRU, Random and Score
                eviction policies (miss counts per step);
  * prefill   - the four-buffer layer pipeline of the prefill: buffer
                bindings, the data it leaves behind, the exposed-time bound.

Every function is pinned by tests under tests/ against values the pages
print, closed forms, special cases and brute force.  Parts without such a pin
are marked "parity unpinned" in their docstring.
"""
from . import formats, indexer, topk, pool, attention, decode, footprint, policies, prefill  # noqa: F401
