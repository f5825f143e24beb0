"""Paged KV-cache attention for AMD MI355X (gfx950).

The KV cache lives in fixed-size physical blocks of one shared pool, reached
through per-sequence block tables. The device work runs in the hand-written
HIP kernels of ``libpagedkv.so`` behind the C ABI of ``include/pagedkv.h``;
this package only marshals torch tensors (device memory, current stream) into
those calls, and wraps the C++ host block allocator.
"""

from ._lib import (AllocatorStateError, OutOfBlocks, PagedKVError, LIB_PATH, SIGNATURES, lib)
from .allocator import BlockAllocator
from .ops import (DecodePlan, KVPool, attention_mixed, cache_write, check_batch, check_chunks,
                  check_copies, check_shared_prefix, check_slots, copy_blocks, decode,
                  decode_noalloc, decode_noalloc_scratch_bytes, decode_shared_prefix,
                  decode_grouped, decode_grouped_workspace_bytes, check_grouped,
                  group_prefix_lens, set_input_checks,
                  decode_shared_prefix_workspace_bytes, decode_workspace_bytes, prefill_chunk,
                  attention_mixed_workspace_bytes,
                  probe_stream_read, swap_blocks, swap_in, swap_out, PA_SWAP_IN, PA_SWAP_OUT)

__all__ = ["AllocatorStateError", "OutOfBlocks", "PagedKVError", "LIB_PATH", "SIGNATURES", "lib",
           "BlockAllocator", "DecodePlan", "KVPool", "attention_mixed", "cache_write", "check_batch",
           "check_chunks", "check_copies", "check_shared_prefix", "check_slots", "copy_blocks",
           "decode", "decode_noalloc", "decode_noalloc_scratch_bytes", "decode_grouped",
           "decode_grouped_workspace_bytes", "check_grouped", "group_prefix_lens",
           "set_input_checks",
           "decode_shared_prefix", "decode_shared_prefix_workspace_bytes",
           "decode_workspace_bytes", "attention_mixed_workspace_bytes", "prefill_chunk", "probe_stream_read", "swap_blocks", "swap_in",
           "swap_out", "PA_SWAP_IN", "PA_SWAP_OUT"]
