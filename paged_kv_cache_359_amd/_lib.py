"""ctypes declarations for libpkv.so (the C ABI in include/pkv.h)."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv.so")

c_i32, c_i64, c_f32, c_sz, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
P_i32 = ctypes.POINTER(ctypes.c_int32)
P_i64 = ctypes.POINTER(ctypes.c_int64)

# name -> (restype, argtypes); mirrors include/pkv.h one to one.
SIGNATURES = {
    "pkv_status_str": (ctypes.c_char_p, [c_i32]),
    "pkv_version": (c_i32, []),
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_alloc_create": (c_i32, [c_i32, c_i32, P_i32, ctypes.POINTER(c_vp)]),
    "pkv_alloc_destroy": (None, [c_vp]),
    "pkv_seq_add": (c_i32, [c_vp, c_i64, c_i32, P_i64]),
    "pkv_seq_add_tokens": (c_i32, [c_vp, c_i64, P_i32, c_i32, P_i64, P_i32]),
    "pkv_seq_fork": (c_i32, [c_vp, c_i64, c_i64]),
    "pkv_seq_append": (c_i32, [c_vp, P_i64, c_i32, P_i64, P_i32, P_i32]),
    "pkv_seq_extend": (c_i32, [c_vp, c_i64, c_i32, P_i64, P_i32, P_i32]),
    "pkv_seq_free": (c_i32, [c_vp, c_i64]),
    "pkv_seq_swap_out": (c_i32, [c_vp, c_i64, c_i32, P_i32, P_i32]),
    "pkv_seq_swap_in": (c_i32, [c_vp, c_i64, c_i32, P_i32, P_i32]),
    "pkv_get_block_tables": (c_i32, [c_vp, P_i64, c_i32, c_i32, P_i32, P_i32]),
    "pkv_seq_length": (c_i32, [c_vp, c_i64, P_i32]),
    "pkv_seq_lengths": (c_i32, [c_vp, P_i64, c_i32, P_i32]),
    "pkv_prefix_groups": (c_i32, [c_vp, P_i64, c_i32, P_i32, P_i32, P_i32]),
    "pkv_shared_prefix_blocks": (c_i32, [c_vp, P_i64, c_i32, P_i32]),
    "pkv_num_free_blocks": (c_i32, [c_vp]),
    "pkv_num_cached_blocks": (c_i32, [c_vp]),
    "pkv_block_refcount": (c_i32, [c_vp, c_i32]),
    "pkv_usage": (c_i32, [c_vp, P_i64, P_i64]),
    "pkv_reshape_and_cache": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32,
                                      c_i32, c_i32, c_vp]),
    "pkv_copy_blocks": (c_i32, [c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp]),
    "pkv_gather_blocks": (c_i32, [c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32,
                                  c_i32, c_vp]),
    "pkv_scatter_blocks": (c_i32, [c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32,
                                   c_i32, c_vp]),
    "pkv_update_block_tables": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32,
                                        c_i32, c_vp]),
    "pkv_append_and_cache": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_vp, c_vp,
                                     c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp]),
    "pkv_decode_workspace_bytes": (c_sz, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32]),
    "pkv_paged_attention_decode": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32,
                                           c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_f32,
                                           c_i32, c_i32, c_vp, c_sz, c_vp]),
    "pkv_paged_attention_decode_noalloc": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32,
                                                   c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                                   c_i32, c_f32, c_i32, c_i32, c_vp]),
    "pkv_cascade_workspace_bytes": (c_sz, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32]),
    "pkv_paged_attention_cascade": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32,
                                            c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                            c_i32, c_f32, c_i32, c_i32, c_vp, c_sz, c_vp]),
    "pkv_paged_attention_prefill": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32,
                                            c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                            c_i32, c_f32, c_i32, c_vp]),
    "pkv_read_probe": (c_i32, [c_vp, c_vp, c_i64, c_i32, c_vp, c_vp]),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load the library once.  Raises if it has not been built: there is no fallback.

    PyTorch is imported first: it maps its own HIP runtime (soname libamdhip64.so.7), and
    the library's dependency on that soname then binds to the same runtime.  Loading the
    library first would map a second HIP/HSA runtime from the ROCm install next to torch's,
    and the two would neither share streams nor, in practice, both see the device.
    """
    global _lib
    if _lib is None:
        import torch  # noqa: F401  (see above: one HIP runtime per process)
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_359_amd.build` "
                "(or __graft_entry__.build()); the paged decode path has no CPU fallback")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib
