"""CPU oracle for paged-KV-cache attention (decode and prefill).

TEST INFRASTRUCTURE ONLY.  This package is the slow, obviously correct,
fp64 definition of what the GPU path computes.  Only the test suite, the
smoke check and the CPU-baseline leg of the benchmark may import it; the
product path (the HIP library and its Python binding) never does, and the
two share no code.

Sources, cited by page title and section:

* "FlashAttention and PagedAttention: two fixes for two different
  bottlenecks" (reactapp.top, es/ru/de), sections "Why attention is
  expensive" (the attention formula), "FlashAttention - How it works"
  (tiling, online softmax, exactness) and "PagedAttention - How it works"
  (fixed-size blocks, per-sequence block table, sharing, a kernel that reads
  scattered blocks through the table).
* "Flash Attention vs Paged Attention" (ewbang.com), section "Paged
  Attention: memory blocking", algorithm principle, eq. (4) (block-wise
  attention over KV blocks) and its memory-management paragraph (blocks fill
  left to right; unfilled slots are reserved).
* "How PagedAttention and RadixAttention optimise KV-cache handling in LLMs"
  (transformaciondigital.pe), section "How PagedAttention works" (the kernel
  consults the table to gather K and V).

Every function here is pinned by tests under ``tests/`` against closed
forms, invariants, brute force and a library routine (torch's CPU
scaled-dot-product attention in float64).  No function is "parity
unpinned".
"""

from . import dtypes  # noqa: F401
from .attention import (  # noqa: F401
    decode,
    decode_row,
    prefill,
    prefill_rows,
    write_kv,
)
