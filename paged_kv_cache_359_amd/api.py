"""Python binding of libpkv.so: argument marshalling only.

Every function here calls the C entry point of the same name (include/pkv.h); all work
happens in the library.  PyTorch supplies device memory and the current HIP stream.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import _lib

PKV_OK = 0
STATUS_NAMES = {0: "PKV_OK", 1: "PKV_ERR_INVALID_ARG", 2: "PKV_ERR_OUT_OF_BLOCKS",
                3: "PKV_ERR_UNKNOWN_SEQ", 4: "PKV_ERR_DUPLICATE_SEQ", 5: "PKV_ERR_UNSUPPORTED",
                6: "PKV_ERR_WORKSPACE", 7: "PKV_ERR_HIP"}
DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2}


class PkvError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = int(status)
        self.name = STATUS_NAMES.get(self.status, str(status))
        detail = ""
        if self.status == 7:
            detail = " (" + _lib.load().pkv_last_error().decode() + ")"
        super().__init__(f"{call}: {self.name}{detail}")


def _check(status: int, call: str):
    if status != PKV_OK:
        raise PkvError(status, call)


def _ptr(arr: np.ndarray, ctype):
    return arr.ctypes.data_as(ctypes.POINTER(ctype))


def pkv_status_str(status: int) -> str:
    return _lib.load().pkv_status_str(int(status)).decode()


def pkv_version() -> int:
    return int(_lib.load().pkv_version())


# ---------------------------------------------------------------------------------------
# Host block allocator
# ---------------------------------------------------------------------------------------
class PkvAlloc:
    """Owns one ``pkv_alloc`` handle; methods map to the ``pkv_seq_*`` / ``pkv_*`` calls."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        self._lib = _lib.load()
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        h = ctypes.c_void_p()
        order = None
        if free_order is not None:
            order = np.ascontiguousarray(free_order, dtype=np.int32)
            if order.shape != (self.num_blocks,):
                raise ValueError("free_order must have num_blocks entries")
        _check(self._lib.pkv_alloc_create(self.num_blocks, self.block_size,
                                          None if order is None else _ptr(order, ctypes.c_int32),
                                          ctypes.byref(h)), "pkv_alloc_create")
        self._h = h

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            self._lib.pkv_alloc_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def pkv_seq_add(self, seq_id: int, num_tokens: int) -> np.ndarray:
        slots = np.empty(max(int(num_tokens), 0), dtype=np.int64)
        _check(self._lib.pkv_seq_add(self._h, int(seq_id), int(num_tokens),
                                     _ptr(slots, ctypes.c_int64) if slots.size else None),
               "pkv_seq_add")
        return slots

    def pkv_seq_add_tokens(self, seq_id: int, tokens):
        """Prefix-cached add: returns (slots int64, n_cached); slots of shared tokens are -1."""
        toks = np.ascontiguousarray(tokens, dtype=np.int32).reshape(-1)
        n = toks.size
        slots = np.empty(max(n, 1), dtype=np.int64)
        nc = ctypes.c_int32(0)
        _check(self._lib.pkv_seq_add_tokens(self._h, int(seq_id), _ptr(toks, ctypes.c_int32) if n else None,
                                            n, _ptr(slots, ctypes.c_int64), ctypes.byref(nc)),
               "pkv_seq_add_tokens")
        return slots[:n], int(nc.value)

    def pkv_seq_fork(self, parent_id: int, child_id: int):
        _check(self._lib.pkv_seq_fork(self._h, int(parent_id), int(child_id)), "pkv_seq_fork")

    def pkv_seq_append(self, seq_ids):
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64).reshape(-1)
        n = ids.size
        slots = np.empty(max(n, 1), dtype=np.int64)
        pairs = np.empty(max(2 * n, 2), dtype=np.int32)
        ncow = ctypes.c_int32(0)
        _check(self._lib.pkv_seq_append(self._h, _ptr(ids, ctypes.c_int64) if n else None, n,
                                        _ptr(slots, ctypes.c_int64), _ptr(pairs, ctypes.c_int32),
                                        ctypes.byref(ncow)), "pkv_seq_append")
        return slots[:n], pairs[: 2 * ncow.value].reshape(-1, 2)

    def pkv_seq_append_into(self, ids: np.ndarray, slots: np.ndarray, pairs: np.ndarray) -> int:
        """Allocation-free variant for hot loops: caller-provided int64 ids/slots and int32
        pairs buffers (2 * n entries).  Returns the number of copy-on-write pairs."""
        ncow = ctypes.c_int32(0)
        _check(self._lib.pkv_seq_append(self._h, _ptr(ids, ctypes.c_int64), ids.size,
                                        _ptr(slots, ctypes.c_int64), _ptr(pairs, ctypes.c_int32),
                                        ctypes.byref(ncow)), "pkv_seq_append")
        return ncow.value

    def pkv_seq_extend(self, seq_id: int, n: int):
        slots = np.empty(max(int(n), 1), dtype=np.int64)
        pairs = np.empty(2, dtype=np.int32)
        ncow = ctypes.c_int32(0)
        _check(self._lib.pkv_seq_extend(self._h, int(seq_id), int(n), _ptr(slots, ctypes.c_int64),
                                        _ptr(pairs, ctypes.c_int32), ctypes.byref(ncow)),
               "pkv_seq_extend")
        return slots[: int(n)], pairs[: 2 * ncow.value].reshape(-1, 2)

    def _swap(self, fn, seq_id, max_blocks):
        blocks = np.empty(max(int(max_blocks), 1), dtype=np.int32)
        n = ctypes.c_int32(0)
        _check(fn(self._h, int(seq_id), int(max_blocks), _ptr(blocks, ctypes.c_int32),
                  ctypes.byref(n)), fn.__name__)
        return blocks[: n.value]

    def pkv_seq_swap_out(self, seq_id: int, max_blocks: int) -> np.ndarray:
        return self._swap(self._lib.pkv_seq_swap_out, seq_id, max_blocks)

    def pkv_seq_swap_in(self, seq_id: int, max_blocks: int) -> np.ndarray:
        return self._swap(self._lib.pkv_seq_swap_in, seq_id, max_blocks)

    def pkv_seq_free(self, seq_id: int):
        _check(self._lib.pkv_seq_free(self._h, int(seq_id)), "pkv_seq_free")

    def pkv_get_block_tables(self, seq_ids, max_blocks: int, tables_out=None, lens_out=None):
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64).reshape(-1)
        n = ids.size
        tables = tables_out if tables_out is not None else np.empty((n, max_blocks), np.int32)
        lens = lens_out if lens_out is not None else np.empty(n, np.int32)
        _check(self._lib.pkv_get_block_tables(self._h, _ptr(ids, ctypes.c_int64) if n else None,
                                              n, int(max_blocks),
                                              _ptr(tables, ctypes.c_int32) if tables.size else None,
                                              _ptr(lens, ctypes.c_int32) if n else None),
               "pkv_get_block_tables")
        return tables, lens

    def pkv_seq_lengths(self, seq_ids, out=None) -> np.ndarray:
        """Lengths of the sequences seq_ids (int32), into ``out`` when given."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64).reshape(-1)
        n = ids.size
        res = out if out is not None else np.empty(n, np.int32)
        _check(self._lib.pkv_seq_lengths(self._h, _ptr(ids, ctypes.c_int64) if n else None, n,
                                         _ptr(res, ctypes.c_int32) if n else None),
               "pkv_seq_lengths")
        return res

    def pkv_shared_prefix_blocks(self, seq_ids, out=None) -> np.ndarray:
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64).reshape(-1)
        n = ids.size
        res = out if out is not None else np.empty(n, np.int32)
        _check(self._lib.pkv_shared_prefix_blocks(self._h, _ptr(ids, ctypes.c_int64) if n else None,
                                                  n, _ptr(res, ctypes.c_int32) if n else None),
               "pkv_shared_prefix_blocks")
        return res

    def pkv_seq_length(self, seq_id: int) -> int:
        out = ctypes.c_int32(0)
        _check(self._lib.pkv_seq_length(self._h, int(seq_id), ctypes.byref(out)), "pkv_seq_length")
        return out.value

    def pkv_prefix_groups(self, seq_ids):
        """(group_start int32 [G + 1], shared_blocks int32 [n]) for cascade decode."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64).reshape(-1)
        n = ids.size
        starts = np.empty(n + 1, dtype=np.int32)
        shared = np.empty(max(n, 1), dtype=np.int32)
        ng = ctypes.c_int32(0)
        _check(self._lib.pkv_prefix_groups(self._h, _ptr(ids, ctypes.c_int64) if n else None, n,
                                           _ptr(starts, ctypes.c_int32), _ptr(shared, ctypes.c_int32),
                                           ctypes.byref(ng)), "pkv_prefix_groups")
        return starts[: ng.value + 1], shared[:n]

    def pkv_num_free_blocks(self) -> int:
        return int(self._lib.pkv_num_free_blocks(self._h))

    def pkv_num_cached_blocks(self) -> int:
        return int(self._lib.pkv_num_cached_blocks(self._h))

    def pkv_block_refcount(self, block: int) -> int:
        return int(self._lib.pkv_block_refcount(self._h, int(block)))

    def pkv_usage(self):
        tok, slots = ctypes.c_int64(0), ctypes.c_int64(0)
        _check(self._lib.pkv_usage(self._h, ctypes.byref(tok), ctypes.byref(slots)), "pkv_usage")
        return tok.value, slots.value


# ---------------------------------------------------------------------------------------
# Device operations (torch tensors on the GPU; launched on the current stream)
# ---------------------------------------------------------------------------------------
def _dtype_code_of(dtype) -> int:
    import torch
    m = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
    if dtype not in m:
        raise TypeError(f"unsupported dtype {dtype}")
    return m[dtype]


def _dtype_code(t) -> int:
    return _dtype_code_of(t.dtype)


def _stream(t) -> int:
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t):
    if not t.is_cuda:
        raise ValueError("expected a GPU tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def pkv_reshape_and_cache(key, value, slot_mapping, k_cache, v_cache):
    """key/value [T, Hkv, D]; slot_mapping [T] int64; caches [N, Hkv, bs, D]."""
    import torch
    if slot_mapping.dtype != torch.int64:
        raise TypeError("slot_mapping must be int64")
    n, hkv, bs, d = k_cache.shape
    t = key.shape[0]
    if key.shape != (t, hkv, d) or value.shape != key.shape or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    if not (key.dtype == value.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("dtype mismatch")
    if slot_mapping.numel() != t:
        raise ValueError("slot_mapping length")
    _check(_lib.load().pkv_reshape_and_cache(
        _dev(key) if t else None, _dev(value) if t else None, _dev(slot_mapping) if t else None,
        _dev(k_cache), _dev(v_cache), t, hkv, d, bs, n, _dtype_code(k_cache), _stream(k_cache)),
        "pkv_reshape_and_cache")


def pkv_copy_blocks(k_cache, v_cache, pairs):
    """pairs: device int32 [n, 2] of (src, dst) block ids."""
    import torch
    if pairs.dtype != torch.int32:
        raise TypeError("pairs must be int32")
    n, hkv, bs, d = k_cache.shape
    npairs = pairs.shape[0] if pairs.numel() else 0
    _check(_lib.load().pkv_copy_blocks(_dev(k_cache), _dev(v_cache),
                                       _dev(pairs) if npairs else None, npairs, hkv, d, bs, n,
                                       _dtype_code(k_cache), _stream(k_cache)), "pkv_copy_blocks")


_HIP = None


def _mapped(t):
    """Device address of a staging buffer: a GPU tensor's own pointer, or for a pinned host
    tensor the address the HIP runtime maps it at on the device (an error if it is not
    mapped)."""
    global _HIP
    if t.is_cuda:
        return _dev(t)
    if not t.is_pinned():
        raise ValueError("staging buffers must be GPU tensors or pinned host tensors")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    if _HIP is None:
        # Looked up through the library's own handle, so the symbol comes from the HIP runtime
        # the library (and torch) is linked against, never from a second copy.
        _HIP = _lib.load()
        _HIP.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p,
                                                 ctypes.c_uint]
        _HIP.hipHostGetDevicePointer.restype = ctypes.c_int
    # The runtime maps whole allocations: map the storage's start and add the view's offset.
    base = t.untyped_storage().data_ptr()
    ptr = ctypes.c_void_p()
    err = _HIP.hipHostGetDevicePointer(ctypes.byref(ptr), ctypes.c_void_p(base), 0)
    if err != 0 or not ptr.value:
        raise ValueError(f"pinned buffer is not mapped for the device (hip error {err})")
    return ptr.value + (t.data_ptr() - base)


def _move_blocks(fn, name, cache_k, cache_v, blocks, buf_k, buf_v):
    import torch
    n, hkv, bs, d = cache_k.shape
    if blocks.dtype != torch.int32:
        raise TypeError("blocks must be int32")
    nb = blocks.numel()
    if buf_k.shape != (nb, hkv, bs, d) or buf_v.shape != buf_k.shape:
        raise ValueError("buffers must be [n_blocks, Hkv, bs, D]")
    if not (buf_k.dtype == buf_v.dtype == cache_k.dtype == cache_v.dtype):
        raise TypeError("dtype mismatch")
    if nb == 0:
        return
    _check(fn(_dev(cache_k), _dev(cache_v), _dev(blocks), nb, _mapped(buf_k), _mapped(buf_v), hkv,
              d, bs, n, _dtype_code(cache_k), _stream(cache_k)), name)


def pkv_gather_blocks(k_cache, v_cache, blocks, k_out, v_out):
    """k_out/v_out [n, Hkv, bs, D] (GPU or pinned host tensors) receive the blocks ``blocks``
    (device int32)."""
    lib = _lib.load()
    _move_blocks(lambda kc, vc, bl, n, kb, vb, *r: lib.pkv_gather_blocks(kc, vc, bl, n, kb, vb, *r),
                 "pkv_gather_blocks", k_cache, v_cache, blocks, k_out, v_out)


def pkv_scatter_blocks(k_in, v_in, blocks, k_cache, v_cache):
    """Blocks ``blocks`` (device int32) of the caches receive k_in/v_in [n, Hkv, bs, D] (GPU or
    pinned host tensors)."""
    lib = _lib.load()
    _move_blocks(lambda kc, vc, bl, n, kb, vb, *r: lib.pkv_scatter_blocks(kb, vb, bl, n, kc, vc, *r),
                 "pkv_scatter_blocks", k_cache, v_cache, blocks, k_in, v_in)


def pkv_update_block_tables(block_tables, context_lens, rows, positions, slot_mapping,
                            block_size: int, num_blocks: int):
    """block_tables [B, max_blocks] int32 and context_lens [B] int32 (device, updated in
    place); rows/positions [n] int32 and slot_mapping [n] int64 (device)."""
    import torch
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    if rows.dtype != torch.int32 or positions.dtype != torch.int32 or slot_mapping.dtype != torch.int64:
        raise TypeError("rows/positions int32, slot_mapping int64")
    n = rows.numel()
    if positions.numel() != n or slot_mapping.numel() != n:
        raise ValueError("rows, positions and slot_mapping differ in length")
    if n == 0:
        return
    _check(_lib.load().pkv_update_block_tables(
        _dev(block_tables), _dev(context_lens), _dev(rows), _dev(positions), _dev(slot_mapping),
        n, block_tables.shape[0], block_tables.shape[1], int(block_size), int(num_blocks),
        _stream(block_tables)), "pkv_update_block_tables")


def pkv_append_and_cache(key, value, slot_mapping, k_cache, v_cache, block_tables=None,
                         context_lens=None, positions=None, rows=None):
    """key/value [n, Hkv, D] (GPU); slot_mapping [n] int64, positions [n] int32 and rows [n]
    int32 (GPU tensors or pinned host tensors, read in place); caches [N, Hkv, bs, D];
    block_tables [B, max_blocks] and context_lens [B] int32 (GPU, updated in place), or both
    None for the cache write alone."""
    import torch
    n, hkv, bs, d = k_cache.shape
    t = key.shape[0]
    if key.shape != (t, hkv, d) or value.shape != key.shape or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    if not (key.dtype == value.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("dtype mismatch")
    if slot_mapping.dtype != torch.int64 or slot_mapping.numel() != t:
        raise ValueError("slot_mapping must be int64 [n]")
    upkeep = block_tables is not None or context_lens is not None
    num_rows = max_blocks = 0
    if upkeep:
        if block_tables is None or context_lens is None or positions is None:
            raise ValueError("block_tables, context_lens and positions go together")
        if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
            raise TypeError("block_tables and context_lens must be int32")
        if block_tables.dim() != 2 or context_lens.shape != (block_tables.shape[0],):
            raise ValueError("table shape")
        if positions.dtype != torch.int32 or positions.numel() != t:
            raise ValueError("positions must be int32 [n]")
        if rows is not None and (rows.dtype != torch.int32 or rows.numel() != t):
            raise ValueError("rows must be int32 [n]")
        num_rows, max_blocks = block_tables.shape
    if t == 0:
        return
    _check(_lib.load().pkv_append_and_cache(
        _dev(key), _dev(value), _mapped(slot_mapping),
        _mapped(rows) if upkeep and rows is not None else None,
        _mapped(positions) if upkeep else None, t, _dev(k_cache), _dev(v_cache),
        _dev(block_tables) if upkeep else None, _dev(context_lens) if upkeep else None,
        num_rows, max_blocks, hkv, d, bs, n, _dtype_code(k_cache), _stream(k_cache)),
        "pkv_append_and_cache")


def pkv_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                               max_context_len, dtype, partition_size=-1) -> int:
    """dtype: "f32" | "f16" | "bf16" or a torch dtype."""
    code = DTYPE_CODES[dtype] if isinstance(dtype, str) else _dtype_code_of(dtype)
    return int(_lib.load().pkv_decode_workspace_bytes(int(num_seqs), int(num_q_heads),
                                                      int(num_kv_heads), int(head_dim),
                                                      int(block_size), int(max_context_len),
                                                      code, int(partition_size)))


def pkv_paged_attention_decode(out, q, k_cache, v_cache, block_tables, context_lens,
                               max_context_len: int, scale: float, partition_size: int = -1,
                               workspace=None, cached_blocks=None):
    """out/q [B, Hq, D]; caches [N, Hkv, bs, D]; block_tables [B, max_blocks] int32;
    context_lens [B] int32; workspace: a uint8 device tensor (or None when none is needed);
    cached_blocks: optional [B] int32 device tensor (cache-policy hint)."""
    import torch
    nb, hq, d = q.shape
    n, hkv, bs, d2 = k_cache.shape
    if d2 != d or out.shape != q.shape or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    if not (q.dtype == out.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("dtype mismatch")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != nb or context_lens.shape != (nb,):
        raise ValueError("table shape")
    cached_ptr = None
    if cached_blocks is not None:
        if cached_blocks.dtype != torch.int32 or cached_blocks.shape != (nb,):
            raise ValueError("cached_blocks must be int32 [num_seqs]")
        cached_ptr = _dev(cached_blocks) if nb else None
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = _dev(workspace), workspace.numel() * workspace.element_size()
    if nb == 0:
        return out
    _check(_lib.load().pkv_paged_attention_decode(
        _dev(out), _dev(q), _dev(k_cache), _dev(v_cache), _dev(block_tables), _dev(context_lens),
        cached_ptr, nb, hq, hkv, d, bs, n, block_tables.shape[1], int(max_context_len),
        float(scale), _dtype_code(k_cache), int(partition_size), ws_ptr, ws_bytes, _stream(q)),
        "pkv_paged_attention_decode")
    return out


PKV_DECODE_SCRATCH_BYTES = 64 << 20  # include/pkv.h


def pkv_paged_attention_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens,
                                       max_context_len: int, scale: float,
                                       partition_size: int = -1, cached_blocks=None):
    """pkv_paged_attention_decode without a workspace: split-K partials go to the library's
    per-GPU scratch array (at most PKV_DECODE_SCRATCH_BYTES); allocates nothing."""
    import torch
    nb, hq, d = q.shape
    n, hkv, bs, d2 = k_cache.shape
    if d2 != d or out.shape != q.shape or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    if not (q.dtype == out.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("dtype mismatch")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != nb or context_lens.shape != (nb,):
        raise ValueError("table shape")
    cached_ptr = None
    if cached_blocks is not None:
        if cached_blocks.dtype != torch.int32 or cached_blocks.shape != (nb,):
            raise ValueError("cached_blocks must be int32 [num_seqs]")
        cached_ptr = _dev(cached_blocks) if nb else None
    if nb == 0:
        return out
    _check(_lib.load().pkv_paged_attention_decode_noalloc(
        _dev(out), _dev(q), _dev(k_cache), _dev(v_cache), _dev(block_tables), _dev(context_lens),
        cached_ptr, nb, hq, hkv, d, bs, n, block_tables.shape[1], int(max_context_len),
        float(scale), _dtype_code(k_cache), int(partition_size), _stream(q)),
        "pkv_paged_attention_decode_noalloc")
    return out


def pkv_cascade_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                max_context_len, dtype, partition_size=-1) -> int:
    """dtype: "f32" | "f16" | "bf16" or a torch dtype."""
    code = DTYPE_CODES[dtype] if isinstance(dtype, str) else _dtype_code_of(dtype)
    return int(_lib.load().pkv_cascade_workspace_bytes(int(num_seqs), int(num_q_heads),
                                                       int(num_kv_heads), int(head_dim),
                                                       int(block_size), int(max_context_len),
                                                       code, int(partition_size)))


def pkv_paged_attention_cascade(out, q, k_cache, v_cache, block_tables, context_lens, group_start,
                                shared_blocks, max_group_size: int, max_context_len: int,
                                scale: float, workspace=None, partition_size: int = -1):
    """As pkv_paged_attention_decode; group_start [G + 1] and shared_blocks [B] are int32
    device tensors (pkv_prefix_groups's output); workspace: None or a uint8 device tensor of
    at least pkv_cascade_workspace_bytes(...) bytes."""
    import torch
    nb, hq, d = q.shape
    n, hkv, bs, d2 = k_cache.shape
    if d2 != d or out.shape != q.shape or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    if not (q.dtype == out.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("dtype mismatch")
    for x in (block_tables, context_lens, group_start, shared_blocks):
        if x.dtype != torch.int32:
            raise TypeError("tables, lengths, group_start and shared_blocks must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != nb or context_lens.shape != (nb,):
        raise ValueError("table shape")
    if shared_blocks.shape != (nb,) or group_start.dim() != 1 or group_start.numel() < 1:
        raise ValueError("group_start [G + 1] and shared_blocks [num_seqs]")
    if nb == 0:
        return out
    ng = group_start.numel() - 1
    _check(_lib.load().pkv_paged_attention_cascade(
        _dev(out), _dev(q), _dev(k_cache), _dev(v_cache), _dev(block_tables), _dev(context_lens),
        _dev(group_start), _dev(shared_blocks), ng, int(max_group_size), nb, hq, hkv, d, bs, n,
        block_tables.shape[1], int(max_context_len), float(scale), _dtype_code(k_cache),
        int(partition_size), _dev(workspace) if workspace is not None and workspace.numel() else None,
        0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(q)), "pkv_paged_attention_cascade")
    return out


def pkv_paged_attention_prefill(out, q, k_cache, v_cache, block_tables, context_lens, query_start,
                                max_query_len: int, max_context_len: int, scale: float):
    """out/q [T, Hq, D]; caches [N, Hkv, bs, D]; block_tables [B, max_blocks] int32;
    context_lens [B] int32 (new tokens included); query_start [B + 1] int32."""
    import torch
    t, hq, d = q.shape
    n, hkv, bs, d2 = k_cache.shape
    nb = context_lens.shape[0]
    if d2 != d or out.shape != q.shape or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    if not (q.dtype == out.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("dtype mismatch")
    for x in (block_tables, context_lens, query_start):
        if x.dtype != torch.int32:
            raise TypeError("block_tables, context_lens and query_start must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != nb or query_start.shape != (nb + 1,):
        raise ValueError("table shape")
    if nb == 0 or t == 0:
        return out
    _check(_lib.load().pkv_paged_attention_prefill(
        _dev(out), _dev(q), _dev(k_cache), _dev(v_cache), _dev(block_tables), _dev(context_lens),
        _dev(query_start), nb, t, hq, hkv, d, bs, n, block_tables.shape[1], int(max_query_len),
        int(max_context_len), float(scale), _dtype_code(k_cache), _stream(q)),
        "pkv_paged_attention_prefill")
    return out


def pkv_read_probe(buf, chunk_bytes: int, checksum, chunk_order=None, num_chunks=None):
    """Reads ``num_chunks`` chunks of ``chunk_bytes`` bytes of the GPU tensor ``buf`` (default:
    all of it) in address order, or in the order ``chunk_order`` (device int32) gives, and
    XORs every 32-bit word read into ``checksum`` (device, one int32/uint32 element)."""
    import torch
    nbytes = buf.numel() * buf.element_size()
    if num_chunks is None:
        num_chunks = nbytes // chunk_bytes
    if num_chunks * chunk_bytes > nbytes:
        raise ValueError("the chunks extend past the end of buf")
    if checksum.dtype not in (torch.int32, torch.uint32) or checksum.numel() < 1:
        raise TypeError("checksum must hold one 32-bit integer")
    order = 0
    if chunk_order is not None:
        if chunk_order.dtype != torch.int32 or chunk_order.numel() != num_chunks:
            raise ValueError("chunk_order must be num_chunks int32")
        order = _dev(chunk_order)
    _check(_lib.load().pkv_read_probe(_dev(buf), order or None, int(num_chunks), int(chunk_bytes),
                                      _dev(checksum), _stream(buf)), "pkv_read_probe")
