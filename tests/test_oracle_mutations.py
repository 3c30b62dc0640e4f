"""Plants plausible mistakes in the CPU oracle and checks that a pin catches each one.

Every mutant is a small, wrong variant of one oracle function, swapped in with monkeypatch
for the duration of one test; the corresponding pins in test_oracle_pins must then fail.
This runs on the CPU only.
"""
import numpy as np
import pytest

import oracle
import oracle.attention as oatt
import oracle.cache as ocache
from tests import test_oracle_pins as pins

FAIL = (AssertionError, IndexError, ValueError)


def _gather_swapped(pool, table, ctx, kv_head):
    bs = pool.shape[2]
    t = np.arange(ctx)
    blocks = np.asarray(table, dtype=np.int64)[np.minimum(t % bs, len(table) - 1)]
    return pool[blocks, kv_head, np.minimum(t // bs, bs - 1), :]


def _attention_keys_as_values(q, keys, values, scale):
    if keys.shape[0] == 0:
        return np.zeros(values.shape[1])
    return oatt.softmax_weights(q, keys, scale) @ keys[:, : values.shape[1]]


def _weights_no_scale(q, keys, scale):
    s = keys @ q
    w = np.exp(s - s.max())
    return w / w.sum()


def _weights_unnormalised(q, keys, scale):
    s = scale * (keys @ q)
    return np.exp(s - s.max())


def _decode_modulo_heads(q_bits, k_pool, v_pool, tables, lens, scale, dtype, num_kv_heads=None):
    q = ocache.to_f64(q_bits, dtype)
    nb, hq, d = q.shape
    hkv = k_pool.shape[1]
    out = np.zeros((nb, hq, d))
    for b in range(nb):
        for h in range(hq):
            g = h % hkv
            k = ocache.to_f64(ocache.gather(k_pool, tables[b], int(lens[b]), g), dtype)
            v = ocache.to_f64(ocache.gather(v_pool, tables[b], int(lens[b]), g), dtype)
            out[b, h] = oatt.attention_contiguous(q[b, h], k, v, scale)
    return out


def _cache_write_transposed(pool, tokens_bits, slots):
    bs = pool.shape[2]
    nb = pool.shape[0]
    for t, s in enumerate(slots):
        if s >= 0:
            pool[(s % bs) % nb, :, (s // bs) % bs, :] = tokens_bits[t]


def _to_f64_bf16_wrong(bits, dtype):
    if dtype == "bf16":
        return (np.asarray(bits).astype(np.uint32) << np.uint32(8)).view(np.float32).astype(float)
    return ORIG_TO_F64(bits, dtype)


ORIG_TO_F64 = ocache.to_f64


def test_gather_index_swap_is_caught(monkeypatch):
    monkeypatch.setattr(oatt, "gather", _gather_swapped)
    with pytest.raises(FAIL):
        pins.test_paged_equals_contiguous_sdpa("tiny", {})


def test_keys_used_as_values_is_caught(monkeypatch):
    monkeypatch.setattr(oatt, "attention_contiguous", _attention_keys_as_values)
    with pytest.raises(FAIL):
        pins.test_brute_force_tiny()


@pytest.mark.parametrize("mutant", [_weights_no_scale, _weights_unnormalised])
def test_softmax_mistakes_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(oatt, "softmax_weights", mutant)
    with pytest.raises(FAIL):
        pins.test_head_mapping_and_scale_against_library()


def test_wrong_gqa_head_mapping_is_caught(monkeypatch):
    monkeypatch.setattr(oracle, "decode", _decode_modulo_heads)
    with pytest.raises(FAIL):
        pins.test_head_mapping_and_scale_against_library()


def test_transposed_cache_write_is_caught(monkeypatch):
    monkeypatch.setattr(oracle, "cache_write", _cache_write_transposed)
    with pytest.raises(FAIL):
        pins.test_cache_round_trip_and_sentinel()


def test_wrong_bf16_upcast_is_caught(monkeypatch):
    monkeypatch.setattr(oracle, "to_f64", _to_f64_bf16_wrong)
    with pytest.raises(FAIL):
        pins.test_upcast_known_values()


class _FifoAllocator(oracle.OracleAllocator):
    def free_seq(self, seq):
        # Freed blocks go to the bottom of the stack (reused last) instead of the top.
        if seq not in self.tables:
            raise oracle.UnknownSeq(seq)
        for b in self.tables[seq]:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.insert(0, b)
        del self.tables[seq]
        del self.lens[seq]


class _NoCowAllocator(oracle.OracleAllocator):
    def append(self, seqs):
        slots = []
        for s in seqs:
            if self.lens[s] % self.block_size == 0:
                self.tables[s].append(self._pop())
            slots.append(self._slot(s))
            self.lens[s] += 1
        return slots, []


def test_fifo_pool_is_caught(monkeypatch):
    monkeypatch.setattr(oracle, "OracleAllocator", _FifoAllocator)
    with pytest.raises(FAIL):
        pins.test_copy_on_write_and_lifo_reuse()


def test_missing_copy_on_write_is_caught(monkeypatch):
    monkeypatch.setattr(oracle, "OracleAllocator", _NoCowAllocator)
    with pytest.raises(FAIL):
        pins.test_copy_on_write_and_lifo_reuse()


def test_reversed_initial_order_is_caught(monkeypatch):
    class Reversed(oracle.OracleAllocator):
        def __init__(self, n, bs, order=None):
            super().__init__(n, bs, order)
            self.free = list(reversed(self.free))
    monkeypatch.setattr(oracle, "OracleAllocator", Reversed)
    with pytest.raises(FAIL):
        pins.test_block_table_7_tokens(pins_golden())


def pins_golden():
    import os
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _prefill_mutant(shift_self=False, positions_from_zero=False):
    def f(q_bits, k_pool, v_pool, tables, ctx_lens, query_start, scale, dtype, num_kv_heads=None):
        q = ocache.to_f64(q_bits, dtype)
        total, hq, d = q.shape
        hkv = k_pool.shape[1]
        out = np.zeros((total, hq, d))
        for b in range(len(ctx_lens)):
            r0, r1 = int(query_start[b]), int(query_start[b + 1])
            n, ctx = r1 - r0, int(ctx_lens[b])
            for g in range(hkv):
                k = ocache.to_f64(ocache.gather(k_pool, tables[b], ctx, g), dtype)
                v = ocache.to_f64(ocache.gather(v_pool, tables[b], ctx, g), dtype)
                for h in range(g * (hq // hkv), (g + 1) * (hq // hkv)):
                    for i in range(n):
                        pos = i if positions_from_zero else ctx - n + i
                        end = pos if shift_self else pos + 1
                        out[r0 + i, h] = oatt.attention_contiguous(q[r0 + i, h], k[:end], v[:end], scale)
        return out
    return f


@pytest.mark.parametrize("kw", [dict(shift_self=True), dict(positions_from_zero=True)])
def test_prefill_mistakes_are_caught(monkeypatch, kw):
    monkeypatch.setattr(oracle, "prefill", _prefill_mutant(**kw))
    with pytest.raises(FAIL):
        pins.test_prefill_on_cached_context_equals_masked_sdpa()
    with pytest.raises(FAIL):
        pins.test_prefill_brute_force_tiny()


# -- prefix caching ----------------------------------------------------------------------
class _LastBlockKeys(dict):
    """A cache that keys a block by its own tokens only, not by the prefix before them."""

    def __init__(self, bs):
        super().__init__()
        self.bs = bs

    def get(self, k, default=None):
        return super().get(k[-self.bs:], default)

    def __setitem__(self, k, v):
        super().__setitem__(k[-self.bs:], v)


class _BlockContentOnly(oracle.OracleAllocator):
    def __init__(self, *a, **kw):
        super().__init__(*a, **kw)
        self.cache = _LastBlockKeys(self.block_size)

    def _restore(self, snap):
        super()._restore(snap)
        c = _LastBlockKeys(self.block_size)
        dict.update(c, self.cache)
        self.cache = c


class _HeadFirstRelease(oracle.OracleAllocator):
    def _release(self, blocks):
        gone = []
        for b in blocks:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                gone.append(b)
        for b in gone:
            (self.evictable if b in self.cached_key else self.free).append(b)


class _HitsStayIdle(oracle.OracleAllocator):
    def add_tokens(self, seq, tokens):
        idle = list(self.evictable)
        out = super().add_tokens(seq, tokens)
        # The shared blocks are put back on the idle list although they are now held.
        self.evictable = [b for b in idle if b in self.evictable or self.ref[b] > 0]
        return out


class _NoRegistration(oracle.OracleAllocator):
    def add_tokens(self, seq, tokens):
        out = super().add_tokens(seq, tokens)
        for b in self.tables[seq]:
            if self.ref[b] == 1 and b in self.cached_key:
                del self.cache[self.cached_key.pop(b)]
        return out


def _prefix_pins():
    from tests import test_oracle_prefix_cache as pc
    return pc


def test_block_content_only_matching_is_caught(monkeypatch):
    pc = _prefix_pins()
    monkeypatch.setattr(oracle, "OracleAllocator", _BlockContentOnly)
    with pytest.raises(FAIL):
        pc.test_sharing_needs_the_whole_prefix()
    with pytest.raises(FAIL):
        pc.test_random_request_streams_read_back_their_own_tokens()


def test_head_first_release_is_caught(monkeypatch):
    monkeypatch.setattr(oracle, "OracleAllocator", _HeadFirstRelease)
    with pytest.raises(FAIL):
        _prefix_pins().test_eviction_order_worked_example()


def test_shared_blocks_left_evictable_are_caught(monkeypatch):
    pc = _prefix_pins()
    monkeypatch.setattr(oracle, "OracleAllocator", _HitsStayIdle)
    with pytest.raises(FAIL):
        pc.test_eviction_order_worked_example_exact()
    with pytest.raises(FAIL):
        pc.test_random_request_streams_read_back_their_own_tokens()


def test_missing_registration_is_caught(monkeypatch):
    monkeypatch.setattr(oracle, "OracleAllocator", _NoRegistration)
    with pytest.raises(FAIL + (oracle.OracleError,)):
        _prefix_pins().test_page_example_by_content(pins_golden())
