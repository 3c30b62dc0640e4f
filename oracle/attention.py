"""Oracle decode attention in float64 — test infrastructure only (see the package docstring).

What it computes.  In autoregressive decoding each new token attends to the keys and values
of every earlier token of its sequence, which are kept in the KV cache ("PagedAttention 与
vLLM 推理加速", §1).  Paging changes only where those keys and values are stored: the kernel
gathers them from scattered physical blocks through the block table, and the result is the
same as with one contiguous buffer — paging is invisible to the model ("vLLM +
PagedAttention：打造高并发LLM推理引擎", steps 3 and 4 under "它是怎么工作的？" and the list
after them; "PagedAttention 与 vLLM 推理加速", §2.3).  So the oracle is the plain definition
of scaled dot-product attention for one query over the gathered, logically ordered K and V,
evaluated in float64 with an explicit two-pass softmax.  It does not reproduce the GPU's
online softmax or its split over partitions; those are the kernel's business, and they must
land on this result.

Prefill (the step before decode on the same cache) processes several new tokens of a
sequence at once.  Every new token still attends to all earlier tokens and to itself, and
to no later one, so row i of a sequence whose newest n tokens are being processed, with ctx
tokens cached after the write, sits at position ctx - n + i and attends to positions
0 .. ctx - n + i ("PagedAttention 与 vLLM 推理加速", §1: each new token sees all previous
tokens).  ``prefill`` writes that definition out row by row; it does not reproduce any
blocking or masking scheme of a kernel.

Readings (also in the design notes):
  * The token appended in a decode step is written to the cache first and attends to itself,
    so a sequence of context length ``ctx`` attends to tokens 0..ctx-1.
  * Grouped-query attention (not on the pages): query head h reads KV head h // G, G = Hq/Hkv.
  * An empty context (ctx == 0) gives an all-zero output.
  * ``scale`` is passed in (1/sqrt(head_dim) in every workload).
"""
from __future__ import annotations

import numpy as np

from .cache import gather, to_f64


def softmax_weights(q: np.ndarray, keys: np.ndarray, scale: float) -> np.ndarray:
    """exp(s_t - max s) / sum_u exp(s_u - max s) with s_t = scale * <q, k_t>, in float64."""
    s = scale * (keys @ q)
    s = s - s.max()
    w = np.exp(s)
    return w / w.sum()


def attention_contiguous(q: np.ndarray, keys: np.ndarray, values: np.ndarray,
                         scale: float) -> np.ndarray:
    """One query [D] over contiguous keys/values [ctx, D] (float64)."""
    if keys.shape[0] == 0:
        return np.zeros(values.shape[1], dtype=np.float64)
    return softmax_weights(q, keys, scale) @ values


def decode(q_bits, k_pool, v_pool, tables, lens, scale: float, dtype: str,
           num_kv_heads: int = None) -> np.ndarray:
    """Paged decode attention for a batch, float64 ``[B, Hq, D]``.

    q_bits   [B, Hq, D] raw bits of the queries (same dtype as the cache)
    k_pool   [N, Hkv, bs, D] raw bits;  v_pool likewise
    tables   [B][max_blocks] physical block ids (entries past the context are unused)
    lens     [B] context lengths
    """
    q = to_f64(q_bits, dtype)
    nb, hq, d = q.shape
    hkv = k_pool.shape[1] if num_kv_heads is None else num_kv_heads
    group = hq // hkv
    out = np.zeros((nb, hq, d), dtype=np.float64)
    for b in range(nb):
        ctx = int(lens[b])
        for g in range(hkv):
            keys = to_f64(gather(k_pool, tables[b], ctx, g), dtype)
            vals = to_f64(gather(v_pool, tables[b], ctx, g), dtype)
            for h in range(g * group, (g + 1) * group):
                out[b, h] = attention_contiguous(q[b, h], keys, vals, scale)
    return out


def prefill(q_bits, k_pool, v_pool, tables, ctx_lens, query_start, scale: float, dtype: str,
            num_kv_heads: int = None) -> np.ndarray:
    """Paged causal prefill attention for a batch, float64 ``[T, Hq, D]``.

    q_bits       [T, Hq, D] raw bits; rows query_start[b] .. query_start[b+1] are the newest
                 n_b tokens of sequence b, in order
    k_pool/v_pool, tables as for ``decode``
    ctx_lens     [B] tokens of each sequence in the cache, the new ones included
    Row i of sequence b attends to positions 0 .. ctx_b - n_b + i.
    """
    q = to_f64(q_bits, dtype)
    total, hq, d = q.shape
    hkv = k_pool.shape[1] if num_kv_heads is None else num_kv_heads
    group = hq // hkv
    out = np.zeros((total, hq, d), dtype=np.float64)
    for b in range(len(ctx_lens)):
        r0, r1 = int(query_start[b]), int(query_start[b + 1])
        n, ctx = r1 - r0, int(ctx_lens[b])
        if n == 0:
            continue
        if n > ctx:
            raise ValueError("more new tokens than cached tokens")
        for g in range(hkv):
            keys = to_f64(gather(k_pool, tables[b], ctx, g), dtype)
            vals = to_f64(gather(v_pool, tables[b], ctx, g), dtype)
            for h in range(g * group, (g + 1) * group):
                for i in range(n):
                    pos = ctx - n + i
                    out[r0 + i, h] = attention_contiguous(q[r0 + i, h], keys[:pos + 1],
                                                          vals[:pos + 1], scale)
    return out
