"""Seeded synthetic inputs for paged decode attention.

This module is shared by the CPU oracle's tests, the GPU path's tests, ``smoke()`` and
``bench.py``.  It only draws random numbers and shapes them into arrays: it contains none of
the method's arithmetic (no block allocation, no slot mapping, no cache write, no attention).
Each side builds its own block tables and caches from these draws.

Workload shapes follow the pages' setting: LLaMA-7B / LLaMA-13B head geometry and 16-token
blocks ("PagedAttention 与 vLLM 推理加速", §1 and §2.2; "vLLM + PagedAttention：打造高并发LLM
推理引擎", the block-size example under "它是怎么工作的？"), mixed context lengths from
continuous batching, grouped-query long contexts and a shared system-prompt prefix
("PagedAttention 与 vLLM 推理加速", §3.2 (3)).

Random streams: ``SeedSequence(1000 + cfg_id).spawn(5)`` gives, in order, the streams for
(context lengths, physical placement, q, k, v).  Lengths and placement use NumPy's PCG64;
q/k/v are drawn N(0, 1) in float32 by a seeded ``torch.Generator`` on the target device and
rounded to the KV dtype by torch's round-to-nearest-even cast.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
DTYPE_SIZE = {"f32": 4, "f16": 2, "bf16": 2}


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    """One decode workload.

    ``lengths`` describes the context length each sequence attends to at its first decode
    step (the cached tokens plus the token appended in that step):
      ("fixed", (l0, l1, ...)) | ("uniform", lo, hi) inclusive |
      ("lognormal", median, sigma, lo, hi) rounded and clipped |
      ("prefix_uniform", lo, hi): a shared prefix of ``prefix_len`` tokens plus a per-sequence
      suffix drawn uniformly in [lo, hi].
    """

    name: str
    cfg_id: int
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    batch: int
    lengths: tuple
    prefix_len: int = 0
    partition_size: int = 512
    steps: int = 1
    # Prefill workloads: how many of each sequence's ``lengths`` tokens are new (processed
    # as one chunk and attending causally); None for decode.  ("all",) = a fresh prompt,
    # ("fixed", n) = a chunk of n tokens on top of cached context.
    new_tokens: Optional[tuple] = None
    # The split-K partition size the workload's description names, if any (timed beside the
    # automatic split).
    stated_partition: Optional[int] = None

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def torch_dtype(self) -> torch.dtype:
        return DTYPES[self.dtype]

    @property
    def dsize(self) -> int:
        return DTYPE_SIZE[self.dtype]


def _cfg5(bs: int, cow: bool) -> DecodeConfig:
    # A 1024-token prefix ends on a block boundary for every swept block size; the
    # copy-on-write variant shortens it by half a block so that the last shared block is
    # partially filled and the first append of each sharer has to copy it.
    prefix = 1024 - (bs // 2 if cow else 0)
    return DecodeConfig(
        name=f"shared_prefix_bs{bs}" + ("_cow" if cow else ""), cfg_id=5, dtype="f16",
        num_q_heads=32, num_kv_heads=32, head_dim=128, block_size=bs,
        num_blocks=131072 // bs, batch=128, lengths=("prefix_uniform", 64, 512),
        prefix_len=prefix)


CONFIGS = {
    # 2 heads, head_dim 8, block 4, 8 physical blocks, contexts 7 and 5, fp32.
    "tiny": DecodeConfig("tiny", 1, "f32", 2, 2, 8, 4, 8, 2, ("fixed", (7, 5))),
    # LLaMA-7B attention shape: 32 heads x 128, bf16 KV, contexts uniform in [128, 2048].
    "llama7b": DecodeConfig("llama7b", 2, "bf16", 32, 32, 128, 16, 16384, 64,
                            ("uniform", 128, 2048)),
    # Prefill (chunked prefill) workloads on the same cache layout.  LLaMA-7B attention shape,
    # 8 fresh prompts of 256..2048 tokens.
    "prefill_llama7b": DecodeConfig("prefill_llama7b", 6, "bf16", 32, 32, 128, 16, 2048, 8,
                                    ("uniform", 256, 2048), new_tokens=("all",)),
    # Grouped-query heads, a 512-token chunk of each of 4 prompts on top of 1024..4096
    # cached tokens.
    "prefill_chunked_gqa": DecodeConfig("prefill_chunked_gqa", 7, "bf16", 64, 8, 128, 16, 2048, 4,
                                        ("uniform", 1536, 4608), new_tokens=("fixed", 512)),
    # LLaMA-13B attention shape: 40 heads x 128, fp16 KV, continuous-batching length mix.
    "llama13b": DecodeConfig("llama13b", 3, "f16", 40, 40, 128, 16, 16384, 256,
                             ("lognormal", 512, 1.0, 16, 4096), steps=64),
    # Grouped-query long context: 64 query heads over 8 KV heads, 32k tokens, split-K.
    "gqa_long": DecodeConfig("gqa_long", 4, "bf16", 64, 8, 128, 16, 33792, 16,
                             ("fixed", (32768,) * 16), stated_partition=512),
}
for _bs in (8, 16, 32):
    for _cow in (False, True):
        _c = _cfg5(_bs, _cow)
        CONFIGS[_c.name] = _c


def get_config(name: str, **overrides) -> DecodeConfig:
    cfg = CONFIGS[name]
    return dataclasses.replace(cfg, **overrides) if overrides else cfg


def seed_streams(cfg_id: int):
    """(lengths, placement, q, k, v) seed sequences for one configuration id."""
    return np.random.SeedSequence(1000 + cfg_id).spawn(5)


def _torch_seed(ss: np.random.SeedSequence) -> int:
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def draw_lengths(cfg: DecodeConfig) -> np.ndarray:
    """Context length attended by each sequence at its first decode step (int64, [batch])."""
    rng = np.random.Generator(np.random.PCG64(seed_streams(cfg.cfg_id)[0]))
    kind = cfg.lengths[0]
    if kind == "fixed":
        vals = np.asarray(cfg.lengths[1], dtype=np.int64)
        full = np.resize(vals, max(cfg.batch, len(vals)))
    elif kind == "uniform":
        lo, hi = cfg.lengths[1], cfg.lengths[2]
        full = rng.integers(lo, hi, size=max(cfg.batch, 1024), endpoint=True)
    elif kind == "lognormal":
        median, sigma, lo, hi = cfg.lengths[1:]
        z = rng.standard_normal(max(cfg.batch, 1024))
        full = np.clip(np.rint(np.exp(np.log(median) + sigma * z)), lo, hi)
    elif kind == "prefix_uniform":
        lo, hi = cfg.lengths[1], cfg.lengths[2]
        full = cfg.prefix_len + rng.integers(lo, hi, size=max(cfg.batch, 1024), endpoint=True)
    else:
        raise ValueError(kind)
    # Drawing a fixed-size stream and slicing keeps a reduced batch a prefix of the full one.
    return np.asarray(full[: cfg.batch], dtype=np.int64)


def new_token_counts(cfg: DecodeConfig, lengths: np.ndarray) -> Optional[np.ndarray]:
    """Tokens of each sequence processed by the prefill step (None for decode workloads)."""
    if cfg.new_tokens is None:
        return None
    kind = cfg.new_tokens[0]
    if kind == "all":
        return lengths.copy()
    if kind == "fixed":
        return np.minimum(lengths, cfg.new_tokens[1]).astype(np.int64)
    raise ValueError(kind)


def draw_free_order(cfg: DecodeConfig) -> np.ndarray:
    """Seeded random permutation of the physical blocks: the order the pool hands them out."""
    rng = np.random.Generator(np.random.PCG64(seed_streams(cfg.cfg_id)[1]))
    return rng.permutation(cfg.num_blocks).astype(np.int32)


_CHUNK = 1 << 22  # elements per draw; fixed so results do not depend on the total size


def draw_normal(shape, seed_seq, dtype: torch.dtype, device) -> torch.Tensor:
    """N(0, 1) float32 draws rounded (RNE) to ``dtype``, drawn in fixed-size chunks."""
    n = int(np.prod(shape)) if len(shape) else 1
    gen = torch.Generator(device=device)
    gen.manual_seed(_torch_seed(seed_seq))
    out = torch.empty(n, dtype=dtype, device=device)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        out[s:e] = torch.randn(e - s, generator=gen, dtype=torch.float32, device=device).to(dtype)
    return out.view(*shape)


@dataclasses.dataclass
class Workload:
    """Everything one side needs to build its caches and run ``cfg.steps`` decode steps.

    Token streams are in logical order.  Sequence ``b`` owns tokens
    ``tok_offsets[b]:tok_offsets[b+1]`` of ``k_tok``/``v_tok``; with a shared prefix those come
    after the ``prefix_len`` tokens of ``k_prefix``/``v_prefix``.  At decode step ``s`` sequence
    ``b`` appends its token number ``lengths[b] - 1 + s`` (counting the prefix) and attends to
    ``lengths[b] + s`` tokens with query ``q[s, b]``.  Prefill workloads instead process the
    newest ``n_new[b]`` of sequence b's ``lengths[b]`` tokens in one step, with queries
    ``q[query_start[b]:query_start[b + 1]]`` ([sum(n_new), Hq, D]).
    """

    cfg: DecodeConfig
    lengths: np.ndarray
    free_order: np.ndarray
    q: torch.Tensor
    k_tok: torch.Tensor
    v_tok: torch.Tensor
    tok_offsets: np.ndarray
    k_prefix: Optional[torch.Tensor]
    v_prefix: Optional[torch.Tensor]
    n_new: Optional[np.ndarray] = None

    @property
    def query_start(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.n_new)]).astype(np.int64)

    @property
    def batch(self) -> int:
        return int(self.lengths.shape[0])

    def token_kv(self, b: int, lo: int, hi: int):
        """K and V of tokens [lo, hi) of sequence b (prefix included), contiguous."""
        p = self.cfg.prefix_len
        if hi <= lo:
            return self.k_tok[:0], self.v_tok[:0]
        ks, vs = [], []
        if lo < p:
            ks.append(self.k_prefix[lo:min(hi, p)])
            vs.append(self.v_prefix[lo:min(hi, p)])
        if hi > p:
            o = int(self.tok_offsets[b])
            a, z = max(lo, p) - p, hi - p
            ks.append(self.k_tok[o + a:o + z])
            vs.append(self.v_tok[o + a:o + z])
        if len(ks) == 1:
            return ks[0], vs[0]
        return torch.cat(ks), torch.cat(vs)


def make_workload(cfg: DecodeConfig, device="cpu") -> Workload:
    lengths = draw_lengths(cfg)
    free_order = draw_free_order(cfg)
    ss = seed_streams(cfg.cfg_id)
    dt = cfg.torch_dtype
    hkv, d = cfg.num_kv_heads, cfg.head_dim
    own = lengths - cfg.prefix_len + (cfg.steps - 1)
    offs = np.zeros(cfg.batch + 1, dtype=np.int64)
    offs[1:] = np.cumsum(own)
    total = int(offs[-1])
    kall = draw_normal((cfg.prefix_len + total, hkv, d), ss[3], dt, device)
    vall = draw_normal((cfg.prefix_len + total, hkv, d), ss[4], dt, device)
    n_new = new_token_counts(cfg, lengths)
    if n_new is None:
        q = draw_normal((cfg.steps, cfg.batch, cfg.num_q_heads, d), ss[2], dt, device)
    else:
        q = draw_normal((int(n_new.sum()), cfg.num_q_heads, d), ss[2], dt, device)
    p = cfg.prefix_len
    return Workload(cfg, lengths, free_order, q, kall[p:], vall[p:], offs,
                    kall[:p] if p else None, vall[:p] if p else None, n_new)


# ---------------------------------------------------------------------------------------
# Request schedule.  What the requests do, in order, to reach their first decode step and
# then to decode: a list of request-level operations that each side replays with its own
# allocator and cache.  Tokens written by an operation are the sequence's next tokens in
# logical order.  ("add", seq, n): a new sequence with n tokens; ("fork", parent, child);
# ("free", seq); ("append", [seq, ...]): one new token for each listed sequence;
# ("extend", seq, n): n new tokens of one sequence (a prefill chunk).
# ---------------------------------------------------------------------------------------
PARENT = -1  # id of the sequence that holds a shared prefix before it is forked


def setup_ops(w: Workload):
    cfg, nb = w.cfg, w.batch
    ops = []
    if cfg.prefix_len:
        ops.append(("add", PARENT, cfg.prefix_len))
        for b in range(nb):
            ops.append(("fork", PARENT, b))
        ops.append(("free", PARENT))
        own = w.lengths - cfg.prefix_len - 1
        for r in range(int(own.max()) if nb else 0):
            ops.append(("append", [b for b in range(nb) if own[b] > r]))
    elif w.n_new is not None:
        for b in range(nb):
            ops.append(("add", b, int(w.lengths[b] - w.n_new[b])))
    else:
        for b in range(nb):
            ops.append(("add", b, int(w.lengths[b]) - 1))
    return ops


def step_ops(w: Workload):
    """One step: every sequence appends the token it decodes, or (prefill) its new chunk."""
    if w.n_new is not None:
        return [("extend", b, int(w.n_new[b])) for b in range(w.batch)]
    return [("append", list(range(w.batch)))]


# -- independently arriving requests that share system prompts ------------------------------
@dataclasses.dataclass(frozen=True)
class PromptStreamConfig:
    """Requests arriving one at a time, each one of ``num_systems`` system prompts followed by
    its own text ("PagedAttention 与 vLLM 推理加速", §3.2 (3): requests with one system prompt
    and different questions).  At most ``live`` requests run at once: when one more arrives,
    the oldest finishes first.  Afterwards the ``live`` remaining requests decode one token.
    System prompt and own lengths are drawn uniformly in the inclusive ranges given."""

    name: str
    cfg_id: int
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    num_requests: int
    num_systems: int
    system_len: tuple
    own_len: tuple
    live: int

    @property
    def torch_dtype(self):
        return DTYPES[self.dtype]

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


PROMPT_STREAMS = {
    # Small enough for the oracle; the pool is tight so idle cached blocks get evicted.
    "prompt_stream_small": PromptStreamConfig("prompt_stream_small", 9, "f16", 8, 4, 128, 16, 96,
                                              40, 3, (20, 200), (1, 60), 6),
    # LLaMA-7B heads, 256 requests over 4 system prompts of 512-2048 tokens.
    "prompt_stream_llama7b": PromptStreamConfig("prompt_stream_llama7b", 10, "f16", 32, 32, 128,
                                                16, 16384, 256, 4, (512, 2048), (16, 512), 64),
}


@dataclasses.dataclass
class PromptStream:
    cfg: PromptStreamConfig
    system_of: np.ndarray      # [R] which system prompt each request starts with
    system_lens: np.ndarray    # [S]
    own_lens: np.ndarray       # [R]
    free_order: np.ndarray     # physical placement (pop order)
    ops: list                  # ("prompt", r) / ("free", r), in arrival order
    live: list                 # requests alive at the end, in arrival order
    sys_k: torch.Tensor        # [S, max system_len, Hkv, D]
    sys_v: torch.Tensor
    own_k: torch.Tensor        # [R, max own_len + 1, Hkv, D]  (+1: the decoded token)
    own_v: torch.Tensor
    q: torch.Tensor            # [len(live), Hq, D]

    def tokens(self, r: int) -> np.ndarray:
        """Token ids of request r's prompt: its system prompt's, then its own (int32)."""
        s = int(self.system_of[r])
        ls, lo = int(self.system_lens[s]), int(self.own_lens[r])
        return np.concatenate([s * 100_000 + np.arange(ls),
                               500_000_000 + r * 100_000 + np.arange(lo)]).astype(np.int32)

    def token_kv(self, r: int, lo: int, hi: int):
        """K/V rows of request r's positions lo .. hi-1 (its system prompt's rows first; the
        position right after the prompt is the decoded token)."""
        s = int(self.system_of[r])
        ls = int(self.system_lens[s])
        ks, vs = [], []
        if lo < ls:
            ks.append(self.sys_k[s, lo:min(hi, ls)])
            vs.append(self.sys_v[s, lo:min(hi, ls)])
        if hi > ls:
            ks.append(self.own_k[r, max(lo, ls) - ls:hi - ls])
            vs.append(self.own_v[r, max(lo, ls) - ls:hi - ls])
        return torch.cat(ks), torch.cat(vs)


def make_prompt_stream(cfg: PromptStreamConfig, device="cpu") -> PromptStream:
    streams = seed_streams(cfg.cfg_id)
    rng = np.random.Generator(np.random.PCG64(streams[0]))
    S, R = cfg.num_systems, cfg.num_requests
    system_lens = rng.integers(cfg.system_len[0], cfg.system_len[1] + 1, size=S)
    system_of = rng.integers(0, S, size=R)
    own_lens = rng.integers(cfg.own_len[0], cfg.own_len[1] + 1, size=R)
    placement = np.random.Generator(np.random.PCG64(streams[1]))
    free_order = placement.permutation(cfg.num_blocks).astype(np.int32)
    ops, alive = [], []
    for r in range(R):
        if len(alive) == cfg.live:
            ops.append(("free", alive.pop(0)))
        ops.append(("prompt", r))
        alive.append(r)
    h, d, dt = cfg.num_kv_heads, cfg.head_dim, DTYPES[cfg.dtype]
    ms, mo = int(system_lens.max()), int(own_lens.max()) + 1
    k = draw_normal((S * ms + R * mo, h, d), streams[3], dt, device)
    v = draw_normal((S * ms + R * mo, h, d), streams[4], dt, device)
    q = draw_normal((len(alive), cfg.num_q_heads, d), streams[2], dt, device)
    return PromptStream(cfg, system_of, system_lens, own_lens, free_order, ops, alive,
                        k[: S * ms].view(S, ms, h, d), v[: S * ms].view(S, ms, h, d),
                        k[S * ms:].view(R, mo, h, d), v[S * ms:].view(R, mo, h, d), q)
