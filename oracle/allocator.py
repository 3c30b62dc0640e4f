"""Oracle block allocator — test infrastructure only (see the package docstring).

What it follows:
  * Fixed-size blocks handed out on demand from one shared pool, one block table per request
    mapping logical page -> physical block, blocks returned to the pool when the request
    ends ("vLLM + PagedAttention：打造高并发LLM推理引擎", the four numbered steps under
    "它是怎么工作的？"; "PagedAttention 与 vLLM 推理加速", §2.2 and §2.3).
  * A request's token n lives in logical page n // block_size at offset n % block_size; the
    physical block comes from the table (same page, §2.3 worked example: 7 tokens with
    4-token blocks occupy pages 0 and 1, and page 1 has one unused slot).
  * Several requests' tables may point at the same physical blocks (shared system prompt),
    kept alive by reference counts; a write to a shared block first copies it
    (copy-on-write) ("PagedAttention 与 vLLM 推理加速", §3.2 (3); "LLM Systems 24: Efficient
    LLM Inference with PagedAttention and vLLM", §3 Conclusion).
  * Running out of blocks is reported to the caller, who may preempt (same §3 Conclusion).

Readings where the pages leave a choice open (each also listed in the design notes):
  * Which free block is used next is not fixed by the pages.  The pool is a LIFO stack whose
    initial pop order is the caller's ``free_order`` (default 0, 1, ..., N-1); freeing a
    sequence walks its table in logical order and pushes each block whose count drops to 0,
    so its last logical block is the first to be reused.
  * ``append`` handles sequences in the order given.  A sequence whose length is a multiple
    of the block size takes a fresh block; otherwise, if its last block is shared
    (count > 1), it takes a fresh block, records the pair (old, new) for the caller to copy,
    and gives up one reference to the old block; a sequence that finds count == 1 writes in
    place.  The slot of the appended token is ``table[-1] * block_size + length %
    block_size``.
  * ``extend`` (several new tokens of one sequence, as a prefill chunk brings) is defined as
    that many single-token appends in a row.
  * Preemption by swapping ("LLM Systems 24", §3 Conclusion: when blocks run out a request
    is preempted and its cache swapped out or recomputed): ``swap_out`` hands the caller the
    sequence's blocks in logical order, then releases them exactly like ``free_seq``;
    ``swap_in`` later takes fresh blocks for all of them, popped in logical order, so the
    restored sequence owns every block (sharing is not re-established).
  * Prefix caching ("PagedAttention 与 vLLM 推理加速", §3.2 (3): requests that share a system
    prompt share its physical blocks; "vLLM 推理加速：PagedAttention、FlashAttention 与动态批处理"
    lists prefix matching, i.e. KV reuse, among a router's signals).  The pages give the
    effect, not the mechanism; the reading here: ``add_tokens`` names a new sequence's
    prompt by its token ids, and each full block of the prompt is identified by the whole
    token prefix that ends with it (the K/V of a position depends on every earlier token).
    The new sequence shares the longest run of leading full blocks whose prefixes are
    cached; its other blocks are fresh, and its fresh full blocks enter the cache.  Cached
    blocks that no sequence holds any more stay cached and "evictable" until their block is
    needed: plain free blocks are used first, then evictable ones, least recently released
    first, a sequence's blocks released tail first.  Evicting a block also makes every cached
    block that extends its prefix unreachable (their content can no longer be found; they
    are evicted in turn when their place in the order comes).
  * Every call either succeeds completely or changes nothing.
"""
from __future__ import annotations

import copy


class OracleError(Exception):
    code = "ERROR"


class InvalidArg(OracleError):
    code = "INVALID_ARG"


class OutOfBlocks(OracleError):
    code = "OUT_OF_BLOCKS"


class UnknownSeq(OracleError):
    code = "UNKNOWN_SEQ"


class DuplicateSeq(OracleError):
    code = "DUPLICATE_SEQ"


class OracleAllocator:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise InvalidArg("num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if free_order is None else [int(x) for x in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise InvalidArg("free_order must be a permutation of range(num_blocks)")
        self.num_blocks = num_blocks
        self.block_size = block_size
        # Top of the stack is the end of the list, so the first pop returns order[0].
        self.free = list(reversed(order))
        self.ref = [0] * num_blocks
        self.tables = {}
        self.lens = {}
        self.swapped = {}  # seq -> (length, number of blocks) while its cache is on the host
        # Prefix cache: token prefix (a tuple ending at a block boundary) -> block, for the
        # reachable entries; every registered block's prefix (reachable or not); and the
        # registered blocks no sequence holds, next to be evicted first.
        self.cache = {}
        self.cached_key = {}
        self.evictable = []

    # -- helpers -----------------------------------------------------------------------
    def _pop(self) -> int:
        if self.free:
            b = self.free.pop()
        elif self.evictable:
            b = self.evictable.pop(0)
            self._evict(b)
        else:
            raise OutOfBlocks("no free block")
        self.ref[b] = 1
        return b

    def _evict(self, b):
        """Drop block b's content from the prefix cache.  If b is where its prefix is found,
        every cached prefix that extends it goes too (those blocks stay registered and
        evictable, but cannot be found).  If b was already unreachable, a newer block may
        hold the same prefix by now, and nothing else changes."""
        key = self.cached_key.pop(b)
        if self.cache.get(key) != b:
            return
        for k in [k for k in self.cache if len(k) >= len(key) and k[:len(key)] == key]:
            del self.cache[k]

    def _release(self, blocks):
        """Drop one reference to each block (a table in logical order).  Blocks reaching 0
        that hold no cached prefix go onto the free stack in logical order; cached ones join
        the evictable order tail first."""
        gone = []
        for b in blocks:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                gone.append(b)
        for b in gone:
            if b not in self.cached_key:
                self.free.append(b)
        for b in reversed(gone):
            if b in self.cached_key:
                self.evictable.append(b)

    def _snapshot(self):
        return (list(self.free), list(self.ref), copy.deepcopy(self.tables), dict(self.lens),
                dict(self.swapped), dict(self.cache), dict(self.cached_key), list(self.evictable))

    def _restore(self, snap):
        (self.free, self.ref, self.tables, self.lens, self.swapped, self.cache,
         self.cached_key, self.evictable) = snap

    def _slot(self, seq) -> int:
        n = self.lens[seq]
        return self.tables[seq][n // self.block_size] * self.block_size + n % self.block_size

    # -- operations --------------------------------------------------------------------
    def add(self, seq, num_tokens: int):
        """New sequence holding ``num_tokens`` tokens; returns their slots in order."""
        if num_tokens < 0:
            raise InvalidArg("num_tokens must be >= 0")
        if seq in self.tables or seq in self.swapped:
            raise DuplicateSeq(seq)
        need = -(-num_tokens // self.block_size)
        if need > self.num_free():
            raise OutOfBlocks(f"need {need} blocks, {self.num_free()} free")
        self.tables[seq] = [self._pop() for _ in range(need)]
        self.lens[seq] = 0
        slots = []
        for _ in range(num_tokens):
            slots.append(self._slot(seq))
            self.lens[seq] += 1
        return slots

    def add_tokens(self, seq, tokens):
        """New sequence whose prompt is the token ids ``tokens``, sharing the cached blocks of
        its longest cached run of leading full-block prefixes.  Returns (slots, n_cached):
        tokens in shared blocks get slot -1 (their K/V is already in the pools) and
        ``n_cached`` counts them; the others get slots in fresh blocks as ``add`` gives."""
        tokens = [int(t) for t in tokens]
        if seq in self.tables or seq in self.swapped:
            raise DuplicateSeq(seq)
        bs = self.block_size
        n = len(tokens)
        hits = []
        for j in range(n // bs):
            b = self.cache.get(tuple(tokens[: (j + 1) * bs]))
            if b is None:
                break
            hits.append(b)
        need = -(-n // bs) - len(hits)
        avail = self.num_free() - sum(1 for b in hits if self.ref[b] == 0)
        if need > avail:
            raise OutOfBlocks(f"need {need} blocks, {avail} free")
        for b in hits:
            if self.ref[b] == 0:
                self.evictable.remove(b)
            self.ref[b] += 1
        table = list(hits)
        for j in range(len(hits), -(-n // bs)):
            b = self._pop()
            table.append(b)
            if (j + 1) * bs <= n:
                key = tuple(tokens[: (j + 1) * bs])
                self.cache[key] = b
                self.cached_key[b] = key
        self.tables[seq] = table
        self.lens[seq] = n
        shared = len(hits) * bs
        slots = [-1 if i < shared else table[i // bs] * bs + i % bs for i in range(n)]
        return slots, shared

    def fork(self, parent, child):
        """``child`` shares every block of ``parent`` (one more reference each)."""
        if parent not in self.tables:
            raise UnknownSeq(parent)
        if child in self.tables or child in self.swapped:
            raise DuplicateSeq(child)
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.ref[b] += 1

    def append(self, seqs):
        """One new token for each sequence, in order.  Returns (slots, cow_pairs)."""
        seqs = list(seqs)
        for s in seqs:
            if s not in self.tables:
                raise UnknownSeq(s)
        if len(set(seqs)) != len(seqs):
            raise InvalidArg("a sequence appears twice in one append")
        snap = self._snapshot()
        slots, pairs = [], []
        try:
            for s in seqs:
                table = self.tables[s]
                if self.lens[s] % self.block_size == 0:
                    table.append(self._pop())
                elif self.ref[table[-1]] > 1:
                    old = table[-1]
                    new = self._pop()
                    self.ref[old] -= 1
                    table[-1] = new
                    pairs.append((old, new))
                slots.append(self._slot(s))
                self.lens[s] += 1
        except OutOfBlocks:
            self._restore(snap)
            raise
        return slots, pairs

    def extend(self, seq, n: int):
        """``n`` new tokens for one sequence (a prefill chunk): the same as ``n`` calls of
        ``append([seq])`` in a row, all or nothing.  Returns (slots, cow_pairs)."""
        if seq not in self.tables:
            raise UnknownSeq(seq)
        if n < 0:
            raise InvalidArg("n must be >= 0")
        snap = self._snapshot()
        slots, pairs = [], []
        try:
            for _ in range(n):
                s, p = self.append([seq])
                slots += s
                pairs += p
        except OutOfBlocks:
            self._restore(snap)
            raise
        return slots, pairs

    def free_seq(self, seq):
        """End a sequence: drop one reference per block; blocks reaching 0 go back."""
        if seq not in self.tables:
            raise UnknownSeq(seq)
        self._release(self.tables[seq])
        del self.tables[seq]
        del self.lens[seq]

    def swap_out(self, seq):
        """Preempt a sequence to host memory: returns its blocks in logical order (the caller
        copies them out first), then gives up its references like ``free_seq`` and remembers
        its length.  Shared blocks stay with their other holders; the host copy is whole."""
        if seq not in self.tables:
            raise UnknownSeq(seq)
        blocks = list(self.tables[seq])
        length = self.lens[seq]
        self.free_seq(seq)
        self.swapped[seq] = (length, len(blocks))
        return blocks

    def swap_in(self, seq):
        """Bring a swapped-out sequence back into fresh blocks, popped in logical order (the
        caller copies its data into them); all or nothing.  Returns the new blocks."""
        if seq not in self.swapped:
            raise UnknownSeq(seq)
        length, nblocks = self.swapped[seq]
        if nblocks > self.num_free():
            raise OutOfBlocks(f"need {nblocks} blocks, {self.num_free()} free")
        self.tables[seq] = [self._pop() for _ in range(nblocks)]
        self.lens[seq] = length
        del self.swapped[seq]
        return list(self.tables[seq])

    # -- queries -----------------------------------------------------------------------
    def prefix_groups(self, seqs):
        """Groups for a decode that reads a shared prefix once per group (cascade attention,
        "LLM Systems 24", §2.2.1.3 names it among runtime-chosen kernels).  A group is a
        maximal run of at least two consecutive rows of ``seqs`` whose tables start with the
        same physical block; it shares the longest common run of leading table entries, cut
        to the full blocks every member's length covers.  Rows in no group (or whose group
        would share nothing) stand alone with 0 shared blocks.
        Returns (group_start [G + 1], shared [n]): rows group_start[g] .. group_start[g+1]-1
        form group g and each shares shared[row] leading blocks."""
        seqs = list(seqs)
        for s in seqs:
            if s not in self.tables:
                raise UnknownSeq(s)
        n, bs = len(seqs), self.block_size
        starts, shared = [0], [0] * n
        i = 0
        while i < n:
            first = self.tables[seqs[i]][:1]
            j = i + 1
            while j < n and first and self.tables[seqs[j]][:1] == first:
                j += 1
            members = [self.tables[seqs[r]] for r in range(i, j)]
            common = 0
            while (j - i >= 2 and all(common < len(t) for t in members)
                   and len({t[common] for t in members}) == 1):
                common += 1
            k = min([common] + [self.lens[seqs[r]] // bs for r in range(i, j)])
            if j - i >= 2 and k > 0:
                shared[i:j] = [k] * (j - i)
                starts.append(j)
            else:
                starts.extend(range(i + 1, j + 1))
            i = j
        return starts, shared

    def block_tables(self, seqs, max_blocks: int):
        """Row-per-sequence tables padded with -1, and the sequence lengths."""
        rows, lens = [], []
        for s in seqs:
            if s not in self.tables:
                raise UnknownSeq(s)
            t = self.tables[s]
            if len(t) > max_blocks:
                raise InvalidArg(f"sequence {s} has {len(t)} blocks > {max_blocks}")
            rows.append(t + [-1] * (max_blocks - len(t)))
            lens.append(self.lens[s])
        return rows, lens

    def num_free(self) -> int:
        """Blocks that can be handed out: free ones and evictable cached ones."""
        return len(self.free) + len(self.evictable)

    def num_cached(self) -> int:
        """Blocks registered in the prefix cache and not evicted (held or evictable)."""
        return len(self.cached_key)

    def refcount(self, block: int) -> int:
        if not 0 <= block < self.num_blocks:
            return -1
        return self.ref[block]

    def usage(self):
        """(tokens stored, slots in allocated blocks); a shared block counts once."""
        tokens = sum(self.lens.values())
        used = sum(1 for r in self.ref if r > 0)
        return tokens, used * self.block_size
