"""Pins the CPU oracle to what the pages and the mathematics fix (no GPU needed).

Each test names what it pins: a worked example the pages print (fixtures under
tests/golden/, each with its citation), a closed form, an invariant, a special case that
reduces to a library routine, or brute force on tiny inputs.  Together they are chosen so
that a plausible mistake in the oracle (a swapped index, the wrong operand, the wrong head
mapping, a dropped scale, a FIFO instead of LIFO pool, a missing copy-on-write) fails one.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
import workloads as W
from tests import oracle_side

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------------------
# Worked examples printed on the pages
# --------------------------------------------------------------------------------------
def test_block_table_7_tokens(golden_dir):
    g = load(golden_dir, "block_table_7_tokens.json")
    a = oracle.OracleAllocator(g["num_blocks"], g["block_size"], g["free_order"])
    slots = a.add("req", g["num_tokens"])
    assert a.tables["req"] == g["expect_table"]
    bs = g["block_size"]
    # Which tokens live on which logical page, and where the table sends that page.
    per_page = [[t for t, s in enumerate(slots) if s // bs == blk] for blk in a.tables["req"]]
    assert per_page == g["expect_tokens_per_page"]
    assert len(a.tables["req"]) * bs - g["num_tokens"] == g["expect_free_slots_in_last_block"]
    # Slot = physical block * block_size + offset (the slot-mapping reading).
    assert slots == [12, 13, 14, 15, 28, 29, 30]


def test_os_paging_interleaved(golden_dir):
    g = load(golden_dir, "os_paging_interleaved.json")
    bs = g["block_size"]
    a = oracle.OracleAllocator(g["num_blocks"], bs, g["free_order"])
    a.add("A", 0)
    a.add("B", 0)
    for _ in range(g["pages_each"]):
        for who in ("A", "B"):
            for _ in range(bs):
                a.append([who])
    assert a.tables["A"] == g["expect_table_A"]
    assert a.tables["B"] == g["expect_table_B"]
    owner = [None] * g["num_blocks"]
    for who in ("A", "B"):
        for blk in a.tables[who]:
            owner[blk] = who
    assert owner == g["expect_owner_by_frame"]
    assert sorted(a.free) == [i for i, o in enumerate(owner) if o is None]


def test_prefix_sharing(golden_dir):
    g = load(golden_dir, "prefix_sharing.json")
    bs = g["block_size"]
    a = oracle.OracleAllocator(g["num_blocks"], bs, g["free_order"])
    a.add("prompt", g["prompt_tokens"])
    reqs = ["r1", "r2", "r3"]
    for r in reqs:
        a.fork("prompt", r)
    a.free_seq("prompt")
    for r, n in zip(reqs, g["suffix_tokens"]):
        for _ in range(n):
            _, pairs = a.append([r])
            assert pairs == []  # the prompt fills whole blocks, so nothing is copied
    assert [a.tables[r] for r in reqs] == g["expect_tables"]
    shared = g["expect_tables"][0][: g["prompt_tokens"] // bs]
    assert all(a.ref[b] == g["expect_refcount_shared"] for b in shared)
    physical = len({b for r in reqs for b in a.tables[r]})
    assert physical == g["expect_physical_blocks"]
    unshared = sum(oracle.calc.blocks_needed(g["prompt_tokens"] + n, bs)
                   for n in g["suffix_tokens"])
    assert unshared == g["expect_unshared_blocks"]
    assert (unshared - physical) == g["expect_saved_blocks_over_prompt_blocks"] * len(shared)
    assert a.num_free() + physical == g["num_blocks"]


def test_contiguous_utilization(golden_dir):
    g = load(golden_dir, "contiguous_utilization.json")
    u = oracle.calc.contiguous_utilization(g["used_tokens"], g["reserved_per_request"])
    assert u == g["expect_utilization"]
    # Paged with 4-token blocks: request 1 fills one block, request 2 half of another.
    assert oracle.calc.paged_utilization(g["used_tokens"], 4) == 6 / 8


def test_kv_cache_size(golden_dir):
    g = load(golden_dir, "kv_cache_size.json")
    n = oracle.calc.kv_cache_bytes(g["layers"], g["heads"], g["head_dim"], g["seq_len"],
                                   g["dtype_size"])
    assert n == 1_677_721_600
    assert round(n / 2 ** 30, 1) == g["expect_gib_one_decimal"]
    # Linear in every factor: doubling the sequence doubles the cache.
    assert oracle.calc.kv_cache_bytes(40, 40, 128, 4096, 2) == 2 * n
    # Per-token, per-layer bytes equal the block formula's per-slot share, over all heads.
    per_block = oracle.calc.block_bytes(16, 128, 128, 40, 2)
    assert per_block * 2048 // 16 * 40 == n


def test_blocks_per_request(golden_dir):
    g = load(golden_dir, "blocks_per_request.json")
    a = oracle.OracleAllocator(64, g["block_size"])
    a.add(0, g["num_tokens"])
    assert len(a.tables[0]) == g["expect_blocks"]
    assert oracle.calc.blocks_needed(g["num_tokens"], g["block_size"]) == g["expect_blocks"]
    # One token more needs one more block.
    a.append([0])
    assert len(a.tables[0]) == g["expect_blocks"] + 1


# --------------------------------------------------------------------------------------
# Allocator invariants
# --------------------------------------------------------------------------------------
def check_invariants(a: oracle.OracleAllocator):
    counts = [0] * a.num_blocks
    for s, t in a.tables.items():
        assert len(t) == oracle.calc.blocks_needed(a.lens[s], a.block_size)
        for b in t:
            counts[b] += 1
    assert counts == a.ref
    free = set(a.free)
    idle = set(a.evictable)
    assert len(free) == len(a.free) and len(idle) == len(a.evictable)
    assert all(a.ref[b] == 0 for b in free | idle)
    referenced = {b for b in range(a.num_blocks) if a.ref[b] > 0}
    assert not (free & referenced) and not (free & idle)
    assert len(free) + len(idle) + len(referenced) == a.num_blocks
    # Cached content: free blocks hold none, idle ones do; a reachable entry's block is
    # registered under that very prefix.
    assert not (free & set(a.cached_key)) and idle <= set(a.cached_key)
    for key, b in a.cache.items():
        assert a.cached_key[b] == key and len(key) % a.block_size == 0


op_strategy = st.lists(
    st.tuples(st.sampled_from(["add", "fork", "append", "free", "swap_out", "swap_in", "extend"]),
              st.integers(0, 5), st.integers(0, 5), st.integers(0, 9)),
    min_size=1, max_size=60)


@settings(max_examples=300, deadline=None)
@given(ops=op_strategy, bs=st.sampled_from([1, 2, 4]), nblocks=st.integers(1, 12),
       seed=st.integers(0, 1000))
def test_allocator_invariants_random_ops(ops, bs, nblocks, seed):
    order = np.random.default_rng(seed).permutation(nblocks)
    a = oracle.OracleAllocator(nblocks, bs, order)
    for kind, x, y, n in ops:
        before = (list(a.free), list(a.ref), {k: list(v) for k, v in a.tables.items()},
                  dict(a.lens), dict(a.swapped))
        try:
            if kind == "add":
                a.add(x, n)
            elif kind == "fork":
                a.fork(x, y)
            elif kind == "free":
                a.free_seq(x)
            elif kind == "extend":
                a.extend(x, n)
            elif kind == "swap_out":
                length, blocks = a.lens.get(x), list(a.tables.get(x, []))
                out = a.swap_out(x)
                assert out == blocks and a.swapped[x] == (length, len(blocks)) and x not in a.tables
            elif kind == "swap_in":
                length, nb = a.swapped.get(x, (None, None))
                new = a.swap_in(x)
                assert len(new) == nb and a.lens[x] == length and all(a.ref[b] == 1 for b in new)
            else:
                seqs = sorted({x, y})
                shared_before = {s: (a.tables[s][-1] if s in a.tables and a.tables[s] else None,
                                     a.ref[a.tables[s][-1]] if s in a.tables and a.tables[s]
                                     else 0) for s in seqs}
                slots, pairs = a.append(seqs)
                for s, slot in zip(seqs, slots):
                    blk = slot // bs
                    # The written block is the sequence's own last block and nobody shares it.
                    assert a.tables[s][-1] == blk and a.ref[blk] == 1
                    assert (a.lens[s] - 1) % bs == slot % bs
                for old, new in pairs:
                    assert a.ref[new] == 1 and a.ref[old] >= 1
                    assert any(shared_before[s][0] == old for s in seqs)
        except oracle.OracleError:
            after = (a.free, a.ref, a.tables, a.lens, a.swapped)
            assert after == before  # failed calls change nothing
        check_invariants(a)


def test_out_of_blocks_is_atomic():
    a = oracle.OracleAllocator(3, 2)
    a.add(0, 2)
    a.add(1, 2)
    # Both sequences need a new block but only one is free.
    with pytest.raises(oracle.OutOfBlocks):
        a.append([0, 1])
    assert a.lens == {0: 2, 1: 2} and a.num_free() == 1 and a.tables == {0: [0], 1: [1]}
    with pytest.raises(oracle.OutOfBlocks):
        a.add(2, 3)
    assert 2 not in a.tables


def test_copy_on_write_and_lifo_reuse():
    a = oracle.OracleAllocator(8, 4, [5, 2, 7, 0, 1, 3, 4, 6])
    a.add("p", 6)                 # blocks 5 (full) and 2 (half)
    a.fork("p", "c")
    assert a.ref[5] == 2 and a.ref[2] == 2
    slots, pairs = a.append(["c"])
    assert pairs == [(2, 7)]      # the shared partial block is copied, not written
    assert a.tables["c"] == [5, 7] and a.tables["p"] == [5, 2]
    assert slots == [7 * 4 + 2]
    slots, pairs = a.append(["p"])  # the parent is now the only owner: writes in place
    assert pairs == [] and slots == [2 * 4 + 2]
    a.free_seq("c")                # 5 stays (parent), 7 goes back
    assert a.free[-1] == 7
    a.free_seq("p")                # pushes 5 then 2: block 2 (last logical) is on top
    assert a.free[-2:] == [5, 2]
    a.add("n", 1)
    assert a.tables["n"] == [2]


# --------------------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,tdt", [("f16", torch.float16), ("bf16", torch.bfloat16)])
def test_upcast_matches_torch_for_every_bit_pattern(dtype, tdt):
    bits = np.arange(1 << 16, dtype=np.uint16)
    ours = oracle.to_f64(bits, dtype)
    ref = torch.from_numpy(bits.view(np.int16)).view(tdt).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_upcast_known_values():
    assert oracle.to_f64(np.array([0x3F80, 0xC000, 0x3F81], np.uint16), "bf16").tolist() == \
        [1.0, -2.0, 1.0078125]
    assert oracle.to_f64(np.array([0x3C00, 0xC000, 0x0001], np.uint16), "f16").tolist() == \
        [1.0, -2.0, 2.0 ** -24]
    assert oracle.to_f64(np.array([0x3F800000], np.uint32), "f32").tolist() == [1.0]


# --------------------------------------------------------------------------------------
# Cache write and gather
# --------------------------------------------------------------------------------------
def test_cache_round_trip_and_sentinel():
    w = W.make_workload(W.get_config("tiny"))
    st_ = oracle_side.build(w, fill=0x7FC00001)  # NaN sentinel in every unused slot
    tables, lens = st_.tables()
    for b in range(w.batch):
        k, v = w.token_kv(b, 0, int(lens[b]))
        for g in range(w.cfg.num_kv_heads):
            kk = oracle.gather(st_.k_pool, tables[b], int(lens[b]), g)
            vv = oracle.gather(st_.v_pool, tables[b], int(lens[b]), g)
            assert np.array_equal(kk, oracle.bits_of(k[:, g], "f32"))
            assert np.array_equal(vv, oracle.bits_of(v[:, g], "f32"))
    used = np.zeros(st_.k_pool.shape[:1] + st_.k_pool.shape[2:3], bool)
    for b in range(w.batch):
        for t in range(int(lens[b])):
            used[tables[b][t // 4], t % 4] = True
    for blk, off in zip(*np.nonzero(~used)):
        assert np.all(st_.k_pool[blk, :, off] == 0x7FC00001)


# --------------------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------------------
def sdpa_f64(q, k, v, scale, gqa=False):
    """torch's scaled_dot_product_attention on the CPU in float64: q [Hq, D], k/v [T, Hkv, D]."""
    qq = torch.from_numpy(q)[:, None, :]             # [Hq, 1, D]
    kk = torch.from_numpy(k).permute(1, 0, 2)        # [Hkv, T, D]
    vv = torch.from_numpy(v).permute(1, 0, 2)
    o = torch.nn.functional.scaled_dot_product_attention(
        qq[None], kk[None].contiguous(), vv[None].contiguous(), scale=scale, enable_gqa=gqa)
    return o[0, :, 0, :].numpy()


def contiguous_f64(w, b, ctx):
    k, v = w.token_kv(b, 0, ctx)
    dt = w.cfg.dtype
    return oracle.to_f64(oracle.bits_of(k, dt), dt), oracle.to_f64(oracle.bits_of(v, dt), dt)


@pytest.mark.parametrize("name,overrides", [
    ("tiny", {}),
    ("llama7b", dict(batch=3, num_blocks=400, num_q_heads=4, num_kv_heads=4)),
    ("gqa_long", dict(batch=2, lengths=("fixed", (70, 33)), num_blocks=40,
                      num_q_heads=16, num_kv_heads=2)),
    ("shared_prefix_bs8_cow", dict(batch=3, num_blocks=600, num_q_heads=2, num_kv_heads=2)),
])
def test_paged_equals_contiguous_sdpa(name, overrides):
    """The paged result equals library attention over the contiguous, unpaged K/V."""
    w = W.make_workload(W.get_config(name, **overrides))
    st_ = oracle_side.build(w)
    out = st_.decode()
    c = w.cfg
    q = oracle.to_f64(oracle.bits_of(w.q[0], c.dtype), c.dtype)
    for b in range(w.batch):
        k, v = contiguous_f64(w, b, int(w.lengths[b]))
        ref = sdpa_f64(q[b], k, v, c.scale, gqa=c.group > 1)
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)


def test_brute_force_tiny():
    """Python loops and math.exp over the tiny workload, token by token."""
    w = W.make_workload(W.get_config("tiny"))
    out = oracle_side.build(w).decode()
    c = w.cfg
    q = oracle.to_f64(oracle.bits_of(w.q[0], c.dtype), c.dtype)
    for b in range(w.batch):
        k, v = contiguous_f64(w, b, int(w.lengths[b]))
        for h in range(c.num_q_heads):
            scores = [c.scale * sum(q[b, h, i] * k[t, h, i] for i in range(c.head_dim))
                      for t in range(k.shape[0])]
            mx = max(scores)
            e = [math.exp(s - mx) for s in scores]
            tot = sum(e)
            ref = [sum(e[t] / tot * v[t, h, i] for t in range(k.shape[0]))
                   for i in range(c.head_dim)]
            np.testing.assert_allclose(out[b, h], ref, rtol=0, atol=1e-13)


def random_case(seed, ctx_list, hq, hkv, d, bs, nblocks):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((len(ctx_list), hq, d)).astype(np.float32)
    kv = [(rng.standard_normal((n, hkv, d)).astype(np.float32),
           rng.standard_normal((n, hkv, d)).astype(np.float32)) for n in ctx_list]
    return q, kv


def paged(q, kv, bs, nblocks, order, scale):
    a = oracle.OracleAllocator(nblocks, bs, order)
    hkv, d = kv[0][0].shape[1:]
    kp = oracle.new_pool(nblocks, hkv, bs, d, "f32")
    vp = oracle.new_pool(nblocks, hkv, bs, d, "f32")
    for b, (k, v) in enumerate(kv):
        slots = a.add(b, k.shape[0])
        oracle.cache_write(kp, k.view(np.uint32), slots)
        oracle.cache_write(vp, v.view(np.uint32), slots)
    mb = max(len(t) for t in a.tables.values()) or 1
    tables, lens = a.block_tables(range(len(kv)), mb)
    return oracle.decode(q.view(np.uint32), kp, vp, tables, lens, scale, "f32")


def test_placement_permutation_is_exact():
    q, kv = random_case(1, [13, 1, 8, 0, 29], 3, 3, 16, 4, 40)
    outs = [paged(q, kv, 4, 40, np.random.default_rng(s).permutation(40), 0.25)
            for s in range(4)]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_shared_blocks_equal_duplicated_blocks():
    bs, d = 4, 8
    rng = np.random.default_rng(7)
    pk = rng.standard_normal((12, 1, d)).astype(np.float32)
    pv = rng.standard_normal((12, 1, d)).astype(np.float32)
    q = rng.standard_normal((2, 1, d)).astype(np.float32)
    # Shared: one copy of the prefix blocks, forked.
    a = oracle.OracleAllocator(16, bs)
    kp = oracle.new_pool(16, 1, bs, d, "f32")
    vp = oracle.new_pool(16, 1, bs, d, "f32")
    s = a.add("p", 12)
    oracle.cache_write(kp, pk.view(np.uint32), s)
    oracle.cache_write(vp, pv.view(np.uint32), s)
    a.fork("p", 0)
    a.fork("p", 1)
    tables, lens = a.block_tables([0, 1], 3)
    assert tables[0] == tables[1]
    shared = oracle.decode(q.view(np.uint32), kp, vp, tables, lens, 0.3, "f32")
    # Duplicated: each sequence writes its own copy.
    dup = paged(q, [(pk, pv), (pk, pv)], bs, 16, None, 0.3)
    assert np.array_equal(shared, dup)


def test_softmax_weights_sum_to_one():
    rng = np.random.default_rng(3)
    for n in (1, 2, 17, 1000, 32768):
        w = oracle.softmax_weights(rng.standard_normal(128), rng.standard_normal((n, 128)),
                                   1 / math.sqrt(128))
        assert abs(w.sum() - 1.0) <= 1e-12 and np.all(w >= 0)


def test_special_cases():
    rng = np.random.default_rng(5)
    d = 32
    v = rng.standard_normal((9, d))
    k = rng.standard_normal((9, d))
    q = rng.standard_normal(d)
    # One token: the output is that token's value row, exactly.
    assert np.array_equal(oracle.attention_contiguous(q, k[:1], v[:1], 0.5), v[0])
    # Zero query or identical keys: uniform weights, the mean of V.
    np.testing.assert_allclose(oracle.attention_contiguous(np.zeros(d), k, v, 0.5),
                               v.mean(0), rtol=0, atol=1e-15)
    same = np.repeat(k[:1], 9, axis=0)
    np.testing.assert_allclose(oracle.attention_contiguous(q, same, v, 0.5), v.mean(0),
                               rtol=0, atol=1e-15)
    # Empty context: zeros.
    assert np.array_equal(oracle.attention_contiguous(q, k[:0], v[:0], 0.5), np.zeros(d))
    # A dominant key selects its value row.
    kk = k.copy()
    kk[4] = q * 100
    np.testing.assert_allclose(oracle.attention_contiguous(q, kk, v, 1.0), v[4], atol=1e-12)


def test_head_mapping_and_scale_against_library():
    """GQA reading h -> h // G and the explicit scale, against torch's GQA attention."""
    q, kv = random_case(11, [21, 6], 8, 2, 16, 4, 20)
    for scale in (0.25, 1.0):
        out = paged(q, kv, 4, 20, None, scale)
        for b, (k, v) in enumerate(kv):
            ref = sdpa_f64(q[b].astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                           scale, gqa=True)
            np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)


def test_block_larger_than_context_is_contiguous():
    q, kv = random_case(2, [5, 3], 2, 2, 8, 8, 4)
    out = paged(q, kv, 8, 4, [3, 1, 0, 2], 0.4)
    for b, (k, v) in enumerate(kv):
        for h in range(2):
            ref = oracle.attention_contiguous(q[b, h].astype(np.float64),
                                              k[:, h].astype(np.float64),
                                              v[:, h].astype(np.float64), 0.4)
            assert np.array_equal(out[b, h], ref)


# --------------------------------------------------------------------------------------
# Prefill: several new tokens per sequence, each attending causally to the cache
# --------------------------------------------------------------------------------------
def paged_prefill(q, kv, n_new, bs, nblocks, order, scale):
    """q [sum(n_new), Hq, D] f32; kv[b] = (k, v) [ctx_b, Hkv, D] f32, the whole cache of
    sequence b after the write; its newest n_new[b] tokens are the queries."""
    a = oracle.OracleAllocator(nblocks, bs, order)
    hkv, d = kv[0][0].shape[1:]
    kp = oracle.new_pool(nblocks, hkv, bs, d, "f32")
    vp = oracle.new_pool(nblocks, hkv, bs, d, "f32")
    for b, (k, v) in enumerate(kv):
        slots = a.add(b, k.shape[0])
        oracle.cache_write(kp, k.view(np.uint32), slots)
        oracle.cache_write(vp, v.view(np.uint32), slots)
    mb = max(len(t) for t in a.tables.values()) or 1
    tables, lens = a.block_tables(range(len(kv)), mb)
    qs = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int64)
    return oracle.prefill(q.view(np.uint32), kp, vp, tables, lens, qs, scale, "f32"), qs


def sdpa_masked_f64(q, k, v, scale, mask=None, causal=False, gqa=False):
    """torch SDPA in float64 on the CPU: q [n, Hq, D], k/v [ctx, Hkv, D] -> [n, Hq, D]."""
    qq = torch.from_numpy(q).permute(1, 0, 2)[None]
    kk = torch.from_numpy(k).permute(1, 0, 2)[None].contiguous()
    vv = torch.from_numpy(v).permute(1, 0, 2)[None].contiguous()
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=m, is_causal=causal,
                                                         scale=scale, enable_gqa=gqa)
    return o[0].permute(1, 0, 2).numpy()


def prefill_case(seed, ctx_list, n_list, hq, hkv, d):
    rng = np.random.default_rng(seed)
    kv = [(rng.standard_normal((c, hkv, d)).astype(np.float32),
           rng.standard_normal((c, hkv, d)).astype(np.float32)) for c in ctx_list]
    q = rng.standard_normal((sum(n_list), hq, d)).astype(np.float32)
    return q, kv


@pytest.mark.parametrize("hq,hkv", [(2, 2), (8, 2)])
def test_prefill_of_a_fresh_prompt_equals_causal_sdpa(hq, hkv):
    """A prompt with no earlier context: row i sees tokens 0..i, torch's is_causal."""
    ctx = [13, 1, 40]
    q, kv = prefill_case(3, ctx, ctx, hq, hkv, 16)
    out, qs = paged_prefill(q, kv, ctx, 4, 40, np.random.default_rng(5).permutation(40), 0.3)
    for b, (k, v) in enumerate(kv):
        ref = sdpa_masked_f64(q[qs[b]:qs[b + 1]].astype(np.float64), k.astype(np.float64),
                              v.astype(np.float64), 0.3, causal=True, gqa=hq != hkv)
        np.testing.assert_allclose(out[qs[b]:qs[b + 1]], ref, rtol=0, atol=1e-12)


def test_prefill_on_cached_context_equals_masked_sdpa():
    """New tokens on top of cached context: row i of n sits at ctx - n + i (explicit mask)."""
    ctx, n_new = [37, 9, 64], [5, 9, 16]
    q, kv = prefill_case(4, ctx, n_new, 6, 3, 8)
    out, qs = paged_prefill(q, kv, n_new, 8, 20, None, 0.5)
    for b, (k, v) in enumerate(kv):
        c, n = ctx[b], n_new[b]
        mask = np.arange(c)[None, :] <= (c - n + np.arange(n))[:, None]
        ref = sdpa_masked_f64(q[qs[b]:qs[b + 1]].astype(np.float64), k.astype(np.float64),
                              v.astype(np.float64), 0.5, mask=mask, gqa=True)
        np.testing.assert_allclose(out[qs[b]:qs[b + 1]], ref, rtol=0, atol=1e-12)


def test_chunked_prefill_equals_one_shot():
    """Splitting a sequence's new tokens into chunks processed one after another (each chunk
    seeing the cache as it stands after its own write) gives the same rows."""
    ctx, n = 50, 30
    q, kv = prefill_case(6, [ctx], [n], 4, 4, 8)
    whole, _ = paged_prefill(q, kv, [n], 4, 16, None, 0.35)
    k, v = kv[0]
    rows = []
    for lo, hi in ((0, 7), (7, 23), (23, 30)):
        c = ctx - n + hi  # cache length after this chunk's write
        part, _ = paged_prefill(q[lo:hi], [(k[:c].copy(), v[:c].copy())], [hi - lo], 4, 16, None, 0.35)
        rows.append(part)
    assert np.array_equal(np.concatenate(rows), whole)


def test_prefill_brute_force_tiny():
    """Python loops and math.exp, token by token, one head."""
    rng = np.random.default_rng(8)
    ctx, n, d = 6, 3, 4
    k = rng.standard_normal((ctx, 1, d)).astype(np.float32)
    v = rng.standard_normal((ctx, 1, d)).astype(np.float32)
    q = rng.standard_normal((n, 1, d)).astype(np.float32)
    out, _ = paged_prefill(q, [(k, v)], [n], 2, 4, [3, 0, 2, 1], 0.7)
    for i in range(n):
        pos = ctx - n + i
        s = [0.7 * sum(float(q[i, 0, e]) * float(k[t, 0, e]) for e in range(d)) for t in range(pos + 1)]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        ref = [sum(w[t] * float(v[t, 0, e]) for t in range(pos + 1)) / sum(w) for e in range(d)]
        np.testing.assert_allclose(out[i, 0], ref, rtol=0, atol=1e-12)


def test_last_prefill_row_equals_decode():
    """The newest row of a prefill is the decode of that sequence at the same length."""
    ctx = [21, 8]
    q, kv = prefill_case(9, ctx, [5, 8], 4, 2, 16)
    out, qs = paged_prefill(q, kv, [5, 8], 4, 20, None, 0.25)
    last = np.stack([q[qs[b + 1] - 1] for b in range(2)])
    dec = paged(last, kv, 4, 20, None, 0.25)
    for b in range(2):
        np.testing.assert_array_equal(out[qs[b + 1] - 1], dec[b])



# --------------------------------------------------------------------------------------
# Swap preemption: a sequence's cache leaves for the host and comes back in fresh blocks
# --------------------------------------------------------------------------------------
def test_swap_round_trip_restores_the_sequence():
    rng = np.random.default_rng(12)
    bs, d, hkv = 4, 8, 2
    a = oracle.OracleAllocator(16, bs, rng.permutation(16))
    kp = oracle.new_pool(16, hkv, bs, d, "f32", fill=0x7FC00001)
    vp = oracle.new_pool(16, hkv, bs, d, "f32", fill=0x7FC00001)
    toks = {}
    for s, n in ((0, 9), (1, 6), (2, 13)):
        k = rng.standard_normal((n, hkv, d)).astype(np.float32)
        v = rng.standard_normal((n, hkv, d)).astype(np.float32)
        slots = a.add(s, n)
        oracle.cache_write(kp, k.view(np.uint32), slots)
        oracle.cache_write(vp, v.view(np.uint32), slots)
        toks[s] = (k, v)
    a.fork(1, 3)  # sequence 1's blocks are shared with 3
    q = rng.standard_normal((4, 2 * hkv, d)).astype(np.float32)

    def dec():
        mb = max(len(t) for t in a.tables.values())
        tables, lens = a.block_tables([0, 1, 2, 3], mb)
        return oracle.decode(q.view(np.uint32), kp, vp, tables, lens, 0.3, "f32")

    ref = dec()
    host = {}
    for s in (1, 0):  # 1 shares its blocks with 3: those stay on the device for 3
        blocks = a.swap_out(s)
        host[s] = (oracle.gather_blocks(kp, blocks), oracle.gather_blocks(vp, blocks))
        check_invariants(a)
    assert 1 not in a.tables and a.swapped[1] == (6, 2)
    with pytest.raises(oracle.DuplicateSeq):
        a.add(1, 3)  # the id is still taken while swapped out
    # Somebody else takes and overwrites the freed blocks meanwhile.
    junk = a.add(9, 4 * (a.num_free() - 5))
    oracle.cache_write(kp, np.zeros((len(junk), hkv, d), np.uint32), junk)
    a.free_seq(9)
    for s in (0, 1):
        new = a.swap_in(s)
        oracle.scatter_blocks(kp, new, host[s][0])
        oracle.scatter_blocks(vp, new, host[s][1])
        check_invariants(a)
    assert a.ref[a.tables[1][0]] == 1  # the restored sequence owns its blocks
    np.testing.assert_array_equal(dec(), ref)
    for s in (0, 1):  # the logical cache reads back token for token
        k, v = toks[s]
        for g in range(hkv):
            got = oracle.gather(kp, a.tables[s], a.lens[s], g)
            assert np.array_equal(got, k[:, g].view(np.uint32))


def test_swap_in_without_room_changes_nothing():
    a = oracle.OracleAllocator(4, 2)
    a.add(0, 5)  # 3 blocks
    a.swap_out(0)
    a.add(1, 4)  # 2 of the 4 blocks
    before = (list(a.free), list(a.ref), dict(a.tables), dict(a.lens), dict(a.swapped))
    with pytest.raises(oracle.OutOfBlocks):
        a.swap_in(0)
    assert (a.free, a.ref, a.tables, a.lens, a.swapped) == before
    a.free_seq(1)
    assert len(a.swap_in(0)) == 3 and a.lens[0] == 5
