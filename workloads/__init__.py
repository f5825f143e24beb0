"""Seeded synthetic inputs for paged KV-cache attention.

This module only draws data: sequence lengths, the free-list order, token ids,
key/value rows, queries, and the script of allocator operations (allocate,
append, fork, free) that a serving loop would issue. It holds none of the
method's arithmetic: no slot rule, no block table, no attention. Both the
library's tests/benchmark and the fp64 oracle read the same draws from here.
"""

import numpy as _np

# Large draws fault in fresh pages; numpy's transparent-hugepage hint makes
# those faults very slow on some sandboxed hosts and buys nothing here.
try:
    _np._core.multiarray._set_madvise_hugepage(False)
except AttributeError:  # older numpy layouts
    pass

from .configs import CONFIGS, config_names, make
from .data import Workload, bf16_bits_to_f32, f32_to_bf16_bits

__all__ = ["CONFIGS", "config_names", "make", "Workload",
           "bf16_bits_to_f32", "f32_to_bf16_bits"]
