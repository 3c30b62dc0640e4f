"""One decode step of a running batch, as a serving loop issues it.

Each step every sequence of the batch gains one token and attends over its whole context
("vLLM + PagedAttention：打造高并发LLM推理引擎", steps 1–3 under "它是怎么工作的？"):

  1. host: the allocator gives each new token its slot, a fresh block when the last one is
     full, or a private copy of a shared, partly filled last block (copy-on-write,
     "PagedAttention 与 vLLM 推理加速", §3.2 (3)); it also reports the tokens' positions and,
     optionally, how many leading blocks each sequence shares with others (a cache hint);
  2. device: the copy-on-write block copies, if any (``pkv_copy_blocks``);
  3. device: ``pkv_append_and_cache`` writes the new K/V into their slots and records each
     token's block and the new length in the block tables and lengths kept on the device;
  4. device: ``pkv_paged_attention_decode`` (plus its partition merge when contexts are
     split).

Every computation is a call into ``libpkv.so``; this class only keeps the buffers they read.
The step's slots and positions are written into pinned host buffers that the append kernel
reads in place, so a step uploads nothing but the copy-on-write pairs (when there are any)
and the hint (when it changed).  ``nbuf`` sets of those buffers rotate; before the host
rewrites a set it waits until the step that last used it is done on the device.  It learns
that from marks, events recorded on the stream after a step's kernels.  Every recorded event
leaves the GPU idle for a few microseconds between the kernels around it, so a mark is
recorded only every ``mark_every`` steps (``mark_every`` <= ``nbuf``, so a mark at or after
the step a set waits for is always there).  Everything is enqueued on the current stream of
the caches' device.
"""
from __future__ import annotations

import collections
import time

import numpy as np

from . import api


class StepMarks:
    """Marks after steps: ``after_step(s)`` records one (an event from ``new_event``) when
    ``every`` steps have passed since the last, or takes the caller's own event, already
    recorded after step s; ``wait_for(s)`` blocks the host until step s's device work is done,
    by waiting on the first mark recorded at or after step s (recording one first if there is
    none)."""

    def __init__(self, new_event, every: int):
        if every < 1:
            raise ValueError("every must be at least 1")
        self._new_event = new_event
        self.every = int(every)
        self._marks = collections.deque()  # (step, event, ours), steps increasing
        self._free = []
        self._last = None  # step of the latest mark
        self._step = -1  # latest step seen by after_step
        self.recorded = 0  # marks recorded here (not the caller's events)

    def _record(self, step):
        e = self._free.pop() if self._free else self._new_event()
        e.record()
        self.recorded += 1
        self._marks.append((step, e, True))
        self._last = step

    def after_step(self, step: int, event=None):
        self._step = step
        if event is not None:
            self._marks.append((step, event, False))
            self._last = step
        elif self._last is None or step - self._last >= self.every:
            self._record(step)

    def wait_for(self, step: int):
        while self._marks and self._marks[0][0] < step:
            _, e, ours = self._marks.popleft()
            if ours:
                self._free.append(e)
        if not self._marks:
            self._record(self._step)
        self._marks[0][1].synchronize()


class DecodeStep:
    """Decode steps over the sequences ``seq_ids`` of ``alloc`` (a ``PkvAlloc``) whose K/V
    live in ``k_cache``/``v_cache`` ([N, Hkv, bs, D] GPU tensors).  ``max_context_len``
    bounds every sequence's length over all the steps to be run (it sizes the device block
    tables and the split-K workspace); ``partition_size`` and ``scale`` are those of
    ``pkv_paged_attention_decode``; ``cache_hint`` passes each sequence's leading blocks
    shared with other sequences as the decode's cached_blocks hint."""

    def __init__(self, alloc, seq_ids, k_cache, v_cache, num_q_heads: int, max_context_len: int,
                 scale: float, partition_size: int = -1, cache_hint: bool = True, nbuf: int = 8,
                 mark_every: int = 4):
        import torch
        dev = k_cache.device
        self.alloc = alloc
        self.ids = np.ascontiguousarray(seq_ids, dtype=np.int64).reshape(-1)
        B = self.ids.size
        n, hkv, bs, d = k_cache.shape
        self.k_cache, self.v_cache = k_cache, v_cache
        self.scale = float(scale)
        self.partition_size = int(partition_size)
        self.max_context_len = int(max_context_len)
        self.max_blocks = max(1, -(-self.max_context_len // bs))
        t, l = alloc.pkv_get_block_tables(self.ids, self.max_blocks)
        if B and int(l.max()) >= self.max_context_len:
            raise ValueError("max_context_len leaves no room for a step")
        self.tables = torch.from_numpy(t).to(dev)
        self.lens = torch.from_numpy(l).to(dev)
        pin = lambda k, dt: torch.empty(max(k, 1), dtype=dt, pin_memory=True)  # noqa: E731
        self.nbuf = int(nbuf)
        self._slots = [pin(B, torch.int64) for _ in range(self.nbuf)]
        self._pos = [pin(B, torch.int32) for _ in range(self.nbuf)]
        self._pairs = [pin(2 * B, torch.int32) for _ in range(self.nbuf)]
        self._hint = [pin(B, torch.int32) for _ in range(self.nbuf)]
        if not 1 <= mark_every <= self.nbuf:
            raise ValueError("mark_every must lie in [1, nbuf]")
        self.marks = StepMarks(torch.cuda.Event, mark_every)
        self.pairs_d = torch.empty((max(B, 1), 2), dtype=torch.int32, device=dev)
        self.hint_d = torch.zeros(max(B, 1), dtype=torch.int32, device=dev) if cache_hint else None
        self._hint_sent = None
        ws = api.pkv_decode_workspace_bytes(max(B, 1), num_q_heads, hkv, d, bs,
                                            self.max_context_len, k_cache.dtype,
                                            self.partition_size)
        self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=dev)
        self.steps = 0
        self.host_seconds = 0.0  # host time of step 1 (allocator calls), summed
        self.cow_copies = 0

    def __call__(self, k_new, v_new, q, out, events=None):
        """One step: k_new/v_new [B, Hkv, D] are the new tokens' K/V, q [B, Hq, D] their
        queries (GPU); the attention output goes to out [B, Hq, D].  ``events``: an optional
        pair of events (``record()``, ``synchronize()``) recorded around the decode call;
        the second then also marks the step's end."""
        B = self.ids.size
        step = self.steps
        i = step % self.nbuf
        self.steps += 1
        if step >= self.nbuf:
            self.marks.wait_for(step - self.nbuf)  # the step that last used this buffer set
        h0 = time.perf_counter()
        pos = self._pos[i].numpy()[:B]
        self.alloc.pkv_seq_lengths(self.ids, pos)
        if B and int(pos.max()) + 1 > self.max_context_len:
            raise ValueError("a sequence outgrows max_context_len")
        ncow = self.alloc.pkv_seq_append_into(self.ids, self._slots[i].numpy()[:B],
                                              self._pairs[i].numpy())
        send_hint = False
        if self.hint_d is not None:
            hint = self._hint[i].numpy()[:B]
            self.alloc.pkv_shared_prefix_blocks(self.ids, hint)
            send_hint = self._hint_sent is None or not np.array_equal(hint, self._hint_sent)
            if send_hint:
                self._hint_sent = hint.copy()
        self.host_seconds += time.perf_counter() - h0
        if send_hint:
            self.hint_d[:B].copy_(self._hint[i][:B], non_blocking=True)
        if ncow:
            self.cow_copies += ncow
            self.pairs_d[:ncow].view(-1).copy_(self._pairs[i][: 2 * ncow], non_blocking=True)
            api.pkv_copy_blocks(self.k_cache, self.v_cache, self.pairs_d[:ncow])
        api.pkv_append_and_cache(k_new, v_new, self._slots[i][:B], self.k_cache, self.v_cache,
                                 self.tables, self.lens, self._pos[i][:B])
        if events is not None:
            events[0].record()
        api.pkv_paged_attention_decode(out, q, self.k_cache, self.v_cache, self.tables, self.lens,
                                       self.max_context_len, self.scale, self.partition_size,
                                       self.workspace,
                                       self.hint_d[:B] if self.hint_d is not None else None)
        # A timing event after the decode serves as this step's mark.
        if events is not None:
            events[1].record()
        self.marks.after_step(step, events[1] if events is not None else None)
        return out
