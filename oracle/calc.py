"""The pages' closed forms — test infrastructure only (see the package docstring)."""
from __future__ import annotations


def kv_cache_bytes(layers: int, heads: int, head_dim: int, seq_len: int, dtype_size: int) -> int:
    """KV-cache size: keys and values (factor 2) for every layer, head, channel and token.

    "PagedAttention 与 vLLM 推理加速", §1 (the KV Cache size equation).
    """
    return 2 * layers * heads * head_dim * seq_len * dtype_size


def block_elements(block_size: int, k_head_dim: int, v_head_dim: int) -> int:
    """Elements in one block for one head of one layer: each of its ``block_size`` tokens
    holds a key and a value row ("PagedAttention 与 vLLM 推理加速", §2.2 block formula; read
    per head and per layer, which the formula leaves implicit)."""
    return block_size * (k_head_dim + v_head_dim)


def block_bytes(block_size: int, k_head_dim: int, v_head_dim: int, kv_heads: int,
                dtype_size: int) -> int:
    """Bytes of one physical block of one layer across all KV heads."""
    return block_elements(block_size, k_head_dim, v_head_dim) * kv_heads * dtype_size


def blocks_needed(num_tokens: int, block_size: int) -> int:
    """Blocks a request of ``num_tokens`` tokens occupies: every full block plus one partly
    filled last block ("PagedAttention 与 vLLM 推理加速", §2.3 and §2.4)."""
    return -(-num_tokens // block_size)


def contiguous_utilization(used_tokens, reserved_per_request: int) -> float:
    """Share of reserved slots in use when every request reserves the same contiguous
    ``reserved_per_request`` slots ("PagedAttention 与 vLLM 推理加速", §2.2 example)."""
    used_tokens = list(used_tokens)
    return sum(used_tokens) / (len(used_tokens) * reserved_per_request)


def paged_utilization(used_tokens, block_size: int) -> float:
    """Share of allocated slots in use with unshared paged blocks (only each request's last
    block can be partly empty)."""
    used_tokens = list(used_tokens)
    return sum(used_tokens) / (sum(blocks_needed(n, block_size) for n in used_tokens) * block_size)
