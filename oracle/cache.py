"""Oracle KV-cache storage — test infrastructure only (see the package docstring).

The cache of one layer is two pools, K and V, of fixed-size blocks shared by all requests
("vLLM 推理加速：PagedAttention、FlashAttention 与动态批处理", the page-pool figure caption under
"Attention vs PagedAttention"; "PagedAttention 与 vLLM 推理加速", §2.2).  A block holds
``block_size`` tokens' keys and values for every KV head (§2.2's block-size formula read per
head and per layer).  Layout of each pool (a reading; the pages fix only the element count):
``[num_blocks, num_kv_heads, block_size, head_dim]``, dense and row-major.

Everything here works on raw bit patterns (uint32 for fp32, uint16 for fp16/bf16) so a cache
write is an exact copy and pools can be compared bit for bit.  Values are only converted, by
``to_f64``, when attention needs them.
"""
from __future__ import annotations

import numpy as np

_BITS = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16}


def bits_of(t, dtype: str) -> np.ndarray:
    """Raw bits of a CPU tensor or array holding ``dtype`` values."""
    if hasattr(t, "detach"):  # torch tensor
        import torch
        t = t.detach().cpu().contiguous()
        view = {"f32": torch.int32, "f16": torch.int16, "bf16": torch.int16}[dtype]
        return t.view(view).numpy().view(_BITS[dtype])
    return np.asarray(t).view(_BITS[dtype])


def to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact conversion of stored bit patterns to float64."""
    bits = np.asarray(bits)
    if dtype == "f32":
        return bits.astype(np.uint32).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        # bfloat16 is the upper half of an IEEE binary32 with the same sign and exponent.
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def new_pool(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int, dtype: str,
             fill: int = 0) -> np.ndarray:
    return np.full((num_blocks, num_kv_heads, block_size, head_dim), fill, dtype=_BITS[dtype])


def cache_write(pool: np.ndarray, tokens_bits: np.ndarray, slots) -> None:
    """Store token t's rows ``[num_kv_heads, head_dim]`` at slot ``slots[t]``; -1 skips.

    Slot s is block ``s // block_size`` at offset ``s % block_size``.
    """
    bs = pool.shape[2]
    slots = np.asarray(slots, dtype=np.int64).reshape(-1)
    keep = np.nonzero(slots >= 0)[0]
    s = slots[keep]
    pool[s // bs, :, s % bs, :] = np.asarray(tokens_bits)[keep]


def copy_blocks(pool: np.ndarray, pairs) -> None:
    """Copy-on-write: whole block ``src`` (all heads, all slots) to block ``dst``."""
    for src, dst in pairs:
        pool[int(dst)] = pool[int(src)]


def gather(pool: np.ndarray, table, ctx: int, kv_head: int) -> np.ndarray:
    """Bits of tokens 0..ctx-1 of one KV head, logically ordered: ``[ctx, head_dim]``.

    Token t is read from physical block ``table[t // block_size]`` at offset
    ``t % block_size`` ("PagedAttention 与 vLLM 推理加速", §2.3).
    """
    bs = pool.shape[2]
    t = np.arange(ctx, dtype=np.int64)
    blocks = np.asarray(table, dtype=np.int64)[t // bs]
    return pool[blocks, kv_head, t % bs, :]


def gather_blocks(pool: np.ndarray, blocks) -> np.ndarray:
    """Whole blocks (every head, every slot) in the given order: ``[n, Hkv, bs, D]`` bits.
    The host copy a swapped-out sequence keeps."""
    return pool[np.asarray(blocks, dtype=np.int64)].copy()


def scatter_blocks(pool: np.ndarray, blocks, data: np.ndarray) -> None:
    """Inverse of ``gather_blocks``: block ``blocks[i]`` receives ``data[i]``."""
    for i, b in enumerate(blocks):
        pool[int(b)] = data[i]
