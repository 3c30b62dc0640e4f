"""Paged KV-cache decode attention for AMD MI355X (gfx950).

The work happens in ``libpkv.so`` (include/pkv.h): a host block allocator and HIP kernels
for the cache write (alone, or fused with the device-side table upkeep of a decode
step), copy-on-write block copies, swap-out/in block moves, paged decode
attention, the split-K partition merge, cascade decode over shared prefixes and paged causal
prefill, and a read-bandwidth probe to rate them against.  This package is its Python binding (argument marshalling only); importing it loads
the library and fails loudly if it has not been built.
"""
from ._lib import load as _load

_load()

from .api import (PkvAlloc, PkvError, pkv_append_and_cache, pkv_copy_blocks, pkv_decode_workspace_bytes,  # noqa: E402
                  pkv_cascade_workspace_bytes, pkv_paged_attention_cascade,
                  pkv_gather_blocks, pkv_scatter_blocks,
                  pkv_paged_attention_decode, pkv_paged_attention_prefill,
                  pkv_read_probe, pkv_reshape_and_cache, pkv_status_str,
                  pkv_update_block_tables, pkv_version, DTYPE_CODES, STATUS_NAMES)

__all__ = ["PkvAlloc", "PkvError", "pkv_append_and_cache", "pkv_copy_blocks", "pkv_decode_workspace_bytes",
           "pkv_cascade_workspace_bytes", "pkv_paged_attention_cascade",
           "pkv_gather_blocks", "pkv_scatter_blocks",
           "pkv_paged_attention_decode", "pkv_paged_attention_prefill",
           "pkv_read_probe", "pkv_reshape_and_cache", "pkv_status_str", "pkv_update_block_tables",
           "pkv_version", "DTYPE_CODES", "STATUS_NAMES"]
