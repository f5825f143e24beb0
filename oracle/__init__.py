"""fp64 CPU oracle for paged KV-cache attention. TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. The library never does: its path runs in the HIP kernels and
fails loudly when they are missing. This package imports nothing from the
library, and the library imports nothing from here; the two share only the
seeded input draws of ``workloads``.

What it computes (the plain definitions, not the GPU algorithm):

* ``attention``: softmax attention of each query against its sequence's
  logical, contiguous keys and values, in float64. The pages state that a
  request sees its KV cache as logically contiguous and that the block table
  only translates addresses ("Why PagedAttention multiplies LLM serving
  throughput", section "Block Table: the GPU page table"; "vLLM PagedAttention
  explained", section 3.3 step 2), so paged attention must equal this.
* ``paging``: a host mirror of the physical block pool, written by the slot
  rule of the block allocator ("LLM inference engine internals", section 2.3,
  ``append_slot``), copied block-wise for copy-on-write, and read back through
  a block table.
* ``allocator``: a reference block manager: FIFO free list, ``allocate`` /
  ``append_slot`` / ``free`` (same page, section 2.3), reference counts and
  copy-on-write ("vLLM PagedAttention explained", sections 4.1 and 4.2), and
  hash-based prefix sharing ("Why PagedAttention multiplies LLM serving
  throughput", section "Automatic prefix caching").
* ``brute``: the same attention in pure-Python loops for tiny inputs.

Pins (tests/test_oracle_*.py, run without a GPU) tie each function to facts
outside itself: the pages' worked examples, closed forms, a library routine
(torch's scaled_dot_product_attention in float64), brute force, and
invariances. No function here is "parity unpinned".
"""

from .attention import decode_attention, prefill_attention
from .allocator import BlockAllocator, OutOfBlocks, AllocatorStateError, run_ops
from .paging import PoolMirror

__all__ = ["decode_attention", "prefill_attention", "BlockAllocator", "OutOfBlocks",
           "AllocatorStateError", "run_ops", "PoolMirror"]
