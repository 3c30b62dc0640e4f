"""Replays a workload's request schedule on the CPU oracle (test infrastructure)."""
from __future__ import annotations

import numpy as np

import oracle
import workloads as W


class OracleState:
    """Oracle allocator plus K/V pools (raw bits) for one workload."""

    def __init__(self, w: W.Workload, free_order=None, fill: int = 0, cache: bool = True):
        c = w.cfg
        self.w = w
        self.cache = cache
        order = w.free_order if free_order is None else free_order
        self.alloc = oracle.OracleAllocator(c.num_blocks, c.block_size, order)
        self.k_pool = self.v_pool = None
        if cache:
            self.k_pool = oracle.new_pool(c.num_blocks, c.num_kv_heads, c.block_size,
                                          c.head_dim, c.dtype, fill)
            self.v_pool = oracle.new_pool(c.num_blocks, c.num_kv_heads, c.block_size,
                                          c.head_dim, c.dtype, fill)
        self.log = []  # (op, slots, cow_pairs) per operation, for comparisons
        self.host = {}  # swapped-out sequence -> (K blocks, V blocks)

    def _write(self, seq, lo, hi, slots):
        if not self.cache:
            return
        b = 0 if seq == W.PARENT else seq
        k, v = self.w.token_kv(b, lo, hi)
        dt = self.w.cfg.dtype
        oracle.cache_write(self.k_pool, oracle.bits_of(k, dt), slots)
        oracle.cache_write(self.v_pool, oracle.bits_of(v, dt), slots)

    def run(self, ops):
        for op in ops:
            kind = op[0]
            if kind == "add":
                _, seq, n = op
                slots = self.alloc.add(seq, n)
                self._write(seq, 0, n, slots)
                self.log.append((op, slots, []))
            elif kind == "fork":
                self.alloc.fork(op[1], op[2])
                self.log.append((op, [], []))
            elif kind == "free":
                self.alloc.free_seq(op[1])
                self.log.append((op, [], []))
            elif kind == "extend":
                _, seq, n = op
                pos = self.alloc.lens[seq]
                slots, pairs = self.alloc.extend(seq, n)
                if self.cache:
                    oracle.copy_blocks(self.k_pool, pairs)
                    oracle.copy_blocks(self.v_pool, pairs)
                self._write(seq, pos, pos + n, slots)
                self.log.append((op, slots, pairs))
            elif kind == "append":
                seqs = op[1]
                pos = [self.alloc.lens[s] for s in seqs]
                slots, pairs = self.alloc.append(seqs)
                if self.cache:
                    oracle.copy_blocks(self.k_pool, pairs)
                    oracle.copy_blocks(self.v_pool, pairs)
                for s, p, sl in zip(seqs, pos, slots):
                    self._write(s, p, p + 1, [sl])
                self.log.append((op, slots, pairs))
            elif kind == "swap_out":
                blocks = self.alloc.swap_out(op[1])
                if self.cache:
                    self.host[op[1]] = (oracle.gather_blocks(self.k_pool, blocks),
                                        oracle.gather_blocks(self.v_pool, blocks))
                self.log.append((op, blocks, []))
            elif kind == "swap_in":
                blocks = self.alloc.swap_in(op[1])
                if self.cache:
                    kb, vb = self.host.pop(op[1])
                    oracle.scatter_blocks(self.k_pool, blocks, kb)
                    oracle.scatter_blocks(self.v_pool, blocks, vb)
                self.log.append((op, blocks, []))
            elif kind == "junk":
                _, seq, n = op
                slots = self.alloc.add(seq, n)
                if self.cache:
                    c = self.w.cfg
                    z = np.zeros((n, c.num_kv_heads, c.head_dim), self.k_pool.dtype)
                    oracle.cache_write(self.k_pool, z, slots)
                    oracle.cache_write(self.v_pool, z, slots)
                self.log.append((op, slots, []))
            else:
                raise ValueError(kind)

    def tables(self, max_blocks=None):
        seqs = list(range(self.w.batch))
        if max_blocks is None:
            max_blocks = max([len(self.alloc.tables[s]) for s in seqs] + [1])
        rows, lens = self.alloc.block_tables(seqs, max_blocks)
        return np.asarray(rows, dtype=np.int32), np.asarray(lens, dtype=np.int32)

    def decode(self, step: int = 0, q_bits=None):
        c = self.w.cfg
        tables, lens = self.tables()
        if q_bits is None:
            q_bits = oracle.bits_of(self.w.q[step], c.dtype)
        return oracle.decode(q_bits, self.k_pool, self.v_pool, tables, lens, c.scale, c.dtype)


    def prefill(self, scale=None):
        c = self.w.cfg
        tables, lens = self.tables()
        q_bits = oracle.bits_of(self.w.q, c.dtype)
        return oracle.prefill(q_bits, self.k_pool, self.v_pool, tables, lens,
                              self.w.query_start, c.scale if scale is None else scale, c.dtype)


def build(w: W.Workload, **kw) -> OracleState:
    st = OracleState(w, **kw)
    st.run(W.setup_ops(w))
    st.run(W.step_ops(w))
    return st
