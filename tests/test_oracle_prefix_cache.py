"""Pins of the oracle's prefix caching (add_tokens), independent of its implementation.

* The pages' worked example of three requests sharing a six-block system prompt
  ("PagedAttention 与 vLLM 推理加速", §3.2 (3)), now with the requests arriving one by one and
  matched by content instead of forked (tests/golden/prefix_sharing.json).
* A hand-worked eviction example of the stated order: plain free blocks first, then idle
  cached blocks in release order, a sequence's blocks tail first.
* Random request streams over a token-valued pool: every live sequence reads back exactly its
  own tokens through its table (no shared block ever holds another prefix, no block is
  handed out while held), a new prompt shares at least the full blocks it has in common with
  any live prompt, every failed call changes nothing, and the block accounting adds up.
"""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from tests.test_oracle_pins import check_invariants


def test_page_example_by_content(golden_dir):
    with open(os.path.join(golden_dir, "prefix_sharing.json")) as f:
        g = json.load(f)
    bs = g["block_size"]
    a = oracle.OracleAllocator(g["num_blocks"], bs, g["free_order"])
    prompt = list(range(1000, 1000 + g["prompt_tokens"]))
    cached = []
    for r, n in enumerate(g["suffix_tokens"]):
        slots, nc = a.add_tokens(r, prompt + [r] * n)
        cached.append(nc)
        # Shared tokens are not written again; the request's own tokens go to its own blocks.
        assert slots[:nc] == [-1] * nc and all(s >= 0 for s in slots[nc:])
    assert cached == [0, g["prompt_tokens"], g["prompt_tokens"]]
    assert [a.tables[r] for r in range(3)] == g["expect_tables"]
    assert all(a.ref[b] == g["expect_refcount_shared"] for b in range(6))
    used = sum(1 for x in a.ref if x > 0)
    assert used == g["expect_physical_blocks"]
    unshared = sum(len(t) for t in g["expect_tables"])
    assert unshared == g["expect_unshared_blocks"]
    assert (unshared - used) == g["expect_saved_blocks_over_prompt_blocks"] * 6
    check_invariants(a)


def test_eviction_order_worked_example():
    # 6 blocks of 2 tokens, handed out 0, 1, 2, ... .
    a = oracle.OracleAllocator(6, 2)
    assert a.add_tokens("A", [1, 2, 3, 4, 5]) == ([0, 1, 2, 3, 4], 0)  # blocks 0, 1 cached; 2 partial
    a.free_seq("A")
    # Block 2 (uncached) is free again; 1 then 0 are idle, tail first.
    assert a.free == [5, 4, 3, 2] and a.evictable == [1, 0] and a.num_free() == 6
    assert a.num_cached() == 2
    a.add("B", 8)  # 4 blocks: the plain free ones 2, 3, 4, 5 first
    assert a.tables["B"] == [2, 3, 4, 5] and a.evictable == [1, 0]
    a.add("C", 1)  # nothing free: evicts block 1, the tail of A's prompt
    assert a.tables["C"] == [1] and a.evictable == [0] and a.num_cached() == 1
    # A's first block is still found, but taking it leaves no block for the third token: the
    # idle block a prompt shares does not also count as free.
    snap = a._snapshot()
    with pytest.raises(oracle.OutOfBlocks):
        a.add_tokens("D", [1, 2, 9])
    assert a._snapshot() == snap
    check_invariants(a)


def test_eviction_order_worked_example_exact():
    a = oracle.OracleAllocator(6, 2)
    a.add_tokens("A", [1, 2, 3, 4, 5])
    a.free_seq("A")
    a.add("B", 8)
    a.add("C", 1)
    a.free_seq("B")  # B's blocks are uncached: back on the free stack, last block on top
    assert a.free == [2, 3, 4, 5]
    slots, nc = a.add_tokens("D", [1, 2, 3, 4])
    # Block 0 (prefix [1, 2]) is found and leaves the idle list; [1, 2, 3, 4] was evicted, so
    # the second block is fresh (5, the top of the free stack) and is registered anew.
    assert nc == 2 and a.tables["D"] == [0, 5] and slots == [-1, -1, 10, 11]
    assert a.evictable == [] and a.num_cached() == 2
    check_invariants(a)


def test_sharing_needs_the_whole_prefix():
    # Equal block contents after different beginnings are different K/V: nothing is shared.
    a = oracle.OracleAllocator(8, 2)
    a.add_tokens(0, [1, 2, 3, 4])
    assert a.add_tokens(1, [9, 9, 3, 4]) == ([4, 5, 6, 7], 0)
    # Same beginning, different second block: only the first block is shared.
    slots, nc = a.add_tokens(2, [1, 2, 5, 6, 7])
    assert nc == 2 and a.tables[2][0] == a.tables[0][0] and a.tables[2][1] != a.tables[0][1]
    check_invariants(a)


def test_add_tokens_out_of_blocks_changes_nothing():
    a = oracle.OracleAllocator(4, 2)
    a.add_tokens(0, [7, 7, 8, 8])
    a.free_seq(0)  # two idle cached blocks, two free
    snap = a._snapshot()
    with pytest.raises(oracle.OutOfBlocks):
        a.add_tokens(1, [7, 7, 8, 8] + [9] * 6)  # shares 2, needs 3 more, only 2 others left
    assert a._snapshot() == snap
    # Sharing both cached blocks leaves exactly the two free ones for the remaining 4 tokens.
    slots, nc = a.add_tokens(1, [7, 7, 8, 8] + [9] * 4)
    assert nc == 4 and a.num_free() == 0
    check_invariants(a)


def lcp_blocks(x, y, bs):
    n = 0
    while n < min(len(x), len(y)) and x[n] == y[n]:
        n += 1
    return n // bs


ops = st.lists(st.tuples(st.sampled_from(["prompt", "prompt", "prompt", "free", "append", "fork",
                                          "swap_out", "swap_in"]),
                         st.integers(0, 5), st.integers(0, 3), st.integers(0, 13)),
               min_size=1, max_size=60)


@settings(max_examples=300, deadline=None)
@given(ops=ops, bs=st.sampled_from([1, 2, 4]), nblocks=st.integers(2, 14),
       seed=st.integers(0, 1000))
def test_random_request_streams_read_back_their_own_tokens(ops, bs, nblocks, seed):
    rng = np.random.default_rng(seed)
    # A few "system prompts" that requests start with, so that prefixes repeat.
    systems = [list(rng.integers(0, 3, size=int(rng.integers(0, 10)))) for _ in range(4)]
    a = oracle.OracleAllocator(nblocks, bs, rng.permutation(nblocks))
    # What each slot holds: a value that stands for the whole token prefix ending at that
    # position, as a position's K/V depends on every token before it.
    pool = np.full(nblocks * bs, -1, dtype=np.int64)
    toks = {}   # live or swapped sequence -> its token ids
    prompts = {}  # sequence created by add_tokens -> its prompt
    host = {}   # swapped-out sequence -> its slots' content
    fresh = [10_000]

    def content(prefix):
        return hash(tuple(prefix))

    def write(slots, p):
        for i, s in enumerate(slots):
            if s >= 0:
                pool[s] = content(p[: i + 1])

    for kind, x, y, n in ops:
        snap = a._snapshot()
        try:
            if kind == "prompt":
                p = systems[y] + [int(t) for t in rng.integers(0, 3, size=n % 7)]
                slots, nc = a.add_tokens(x, p)
                assert nc % bs == 0 and slots[:nc] == [-1] * nc and min(slots[nc:], default=0) >= 0
                for s2, p2 in prompts.items():
                    if s2 in a.tables and s2 != x:
                        assert nc >= lcp_blocks(p, p2, bs) * bs
                assert a.lens[x] == len(p) and len(a.tables[x]) == -(-len(p) // bs)
                write(slots, p)
                toks[x] = [content(p[: i + 1]) for i in range(len(p))]
                prompts[x] = list(p)
            elif kind == "free":
                a.free_seq(x)
                toks.pop(x)
                prompts.pop(x, None)
            elif kind == "append":
                seqs = sorted({x, y})
                slots, pairs = a.append(seqs)
                for old, new in pairs:
                    pool[new * bs:(new + 1) * bs] = pool[old * bs:(old + 1) * bs]
                for s, slot in zip(seqs, slots):
                    fresh[0] += 1
                    pool[slot] = fresh[0]
                    toks[s].append(fresh[0])
            elif kind == "fork":
                a.fork(x, y)
                toks[y] = list(toks[x])
            elif kind == "swap_out":
                blocks = a.swap_out(x)
                host[x] = [pool[b * bs:(b + 1) * bs].copy() for b in blocks]
                prompts.pop(x, None)
            else:
                blocks = a.swap_in(x)
                for b, data in zip(blocks, host.pop(x)):
                    pool[b * bs:(b + 1) * bs] = data
        except oracle.OracleError:
            assert a._snapshot() == snap
        check_invariants(a)
        for s, t in a.tables.items():
            got = [int(pool[t[i // bs] * bs + i % bs]) for i in range(a.lens[s])]
            assert got == toks[s], (kind, s)
        used = sum(1 for r in a.ref if r > 0)
        assert used + a.num_free() == nblocks


# -- cascade groups -------------------------------------------------------------------------
def test_prefix_groups_page_example(golden_dir):
    # The pages' three requests forked from one six-block prompt form one group sharing it.
    with open(os.path.join(golden_dir, "prefix_sharing.json")) as f:
        g = json.load(f)
    bs = g["block_size"]
    a = oracle.OracleAllocator(g["num_blocks"], bs, g["free_order"])
    a.add("p", g["prompt_tokens"])
    for r in range(3):
        a.fork("p", r)
    a.free_seq("p")
    for r, n in enumerate(g["suffix_tokens"]):
        for _ in range(n):
            a.append([r])
    assert a.prefix_groups([0, 1, 2]) == ([0, 3], [6, 6, 6])
    # Reordered rows form the same group; a single row shares nothing with itself.
    assert a.prefix_groups([2, 0]) == ([0, 2], [6, 6])
    assert a.prefix_groups([1]) == ([0, 1], [0])


def test_prefix_groups_worked_example():
    a = oracle.OracleAllocator(32, 4)
    a.add("x", 8)          # blocks 0, 1
    a.fork("x", "x2")
    a.add("solo", 3)       # block 2
    a.add("y", 10)         # blocks 3, 4, 5 (last one partial)
    a.fork("y", "y2")
    a.fork("y", "y3")
    a.append(["y2"])       # y2 copies block 5 on write: y, y3 still share it
    a.add("short", 0)
    # Rows: x, x2 | solo | y, y2, y3 | short | x  (x again, not next to x2)
    starts, shared = a.prefix_groups(["x", "x2", "solo", "y", "y2", "y3", "short", "x"])
    assert starts == [0, 2, 3, 6, 7, 8]
    # x/x2 share both blocks (8 tokens = 2 full blocks).  y, y2, y3 share blocks 3 and 4
    # (block 5 differs for y2), and 10 // 4 = 2 full blocks anyway.
    assert shared == [2, 2, 0, 2, 2, 2, 0, 0]
    a.fork("y", "y4")  # y and y4 share block 5 too, but it is not full: cut to 2
    assert a.prefix_groups(["y", "y4"]) == ([0, 2], [2, 2])


@settings(max_examples=200, deadline=None)
@given(ops=st.lists(st.tuples(st.sampled_from(["add", "fork", "fork", "append", "free"]),
                              st.integers(0, 5), st.integers(0, 5), st.integers(0, 12)),
                    min_size=1, max_size=40),
       bs=st.sampled_from([1, 2, 4]), seed=st.integers(0, 100))
def test_prefix_groups_properties(ops, bs, seed):
    a = oracle.OracleAllocator(64, bs, np.random.default_rng(seed).permutation(64))
    for kind, x, y, n in ops:
        try:
            {"add": lambda: a.add(x, n), "fork": lambda: a.fork(x, y),
             "append": lambda: a.append([x]), "free": lambda: a.free_seq(x)}[kind]()
        except oracle.OracleError:
            pass
    rows = sorted(a.tables, key=lambda s: (a.tables[s][:1], s))
    starts, shared = a.prefix_groups(rows)
    assert starts[0] == 0 and starts[-1] == len(rows) and starts == sorted(set(starts))
    for g0, g1 in zip(starts, starts[1:]):
        tabs = [a.tables[rows[r]] for r in range(g0, g1)]
        k = shared[g0]
        assert all(shared[r] == k for r in range(g0, g1))
        if g1 - g0 == 1:
            assert k == 0
            continue
        assert k > 0 and all(t[:k] == tabs[0][:k] for t in tabs)  # the same physical blocks
        assert all(a.lens[rows[r]] >= k * bs for r in range(g0, g1))  # full for every member
        longer = all(len(t) > k for t in tabs) and len({t[k] for t in tabs}) == 1
        assert not longer or any(a.lens[rows[r]] < (k + 1) * bs for r in range(g0, g1))
    for r in range(len(rows) - 1):  # runs are maximal
        if r + 1 not in starts[1:-1]:
            continue
        t0, t1 = a.tables[rows[r]][:1], a.tables[rows[r + 1]][:1]
        assert not t0 or t0 != t1 or shared[r] == 0 or shared[r + 1] == 0
