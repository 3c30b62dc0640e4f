"""CPU oracle for paged decode attention — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct CPU implementation of what the GPU path computes, written
from the pages and checked against what they fix (worked examples, closed forms, invariants,
library special cases; see ``tests/test_oracle_pins.py``).  Only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import it.  It shares
no code with the HIP library: the two meet only at the seeded inputs of ``workloads.py``.

Modules:
  allocator  block pool, per-sequence block tables, reference counts, copy-on-write,
             slot mapping (pure Python lists and dicts)
  cache      cache write, block copy and gather on raw bit patterns (NumPy)
  attention  decode and causal prefill attention in float64 by their plain definition (NumPy)
  calc       the pages' closed forms: KV-cache size, block size, utilisation
"""
from .allocator import (OracleAllocator, OracleError, OutOfBlocks, UnknownSeq, DuplicateSeq,
                        InvalidArg)
from .cache import (new_pool, cache_write, copy_blocks, gather, gather_blocks, scatter_blocks,
                    to_f64, bits_of)
from .attention import decode, prefill, attention_contiguous, softmax_weights
from . import calc

__all__ = [
    "OracleAllocator", "OracleError", "OutOfBlocks", "UnknownSeq", "DuplicateSeq", "InvalidArg",
    "new_pool", "cache_write", "copy_blocks", "gather", "gather_blocks", "scatter_blocks",
    "to_f64", "bits_of",
    "decode", "prefill", "attention_contiguous", "softmax_weights", "calc",
]
