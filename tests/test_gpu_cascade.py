"""Cascade decode on the GPU against the oracle's plain attention.

The cascade reads each group's shared prefix once per 16 (member, query head) columns on
matrix cores, then each member's own blocks with only that member's columns taking part.  It
computes the same quantity as plain paged decode, so the bar is the attention bar against
the fp64 oracle (and the plain decode must meet it too).  Groups come from
pkv_prefix_groups on the library's allocator.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
import paged_kv_cache_359_amd as pkv
from tests import gpu_side, oracle_side
from tests.tolerance import check

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def cascade(alloc, rows, q, k_cache, v_cache, scale, partition_size=-1, max_group_size=None,
            shared_override=None):
    """Runs the cascade for batch rows ``rows`` (in that order) and returns (out, groups)."""
    n, hkv, bs, d = k_cache.shape
    starts, shared = alloc.pkv_prefix_groups(rows)
    tables, lens = alloc.pkv_get_block_tables(rows, max(-(-int(l) // bs) for l in
                                                        [alloc.pkv_seq_length(r) for r in rows]))
    mc = int(lens.max())
    nb, hq, _ = q.shape
    ws_n = pkv.pkv_cascade_workspace_bytes(nb, hq, hkv, d, bs, mc, q.dtype, partition_size)
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda") if ws_n else None
    out = torch.empty_like(q)
    gsz = int(np.max(np.diff(starts))) if starts.size > 1 else 0
    if max_group_size is not None:
        gsz = max_group_size
    sh = shared if shared_override is None else shared_override
    pkv.pkv_paged_attention_cascade(out, q, k_cache, v_cache, torch.from_numpy(tables).cuda(),
                                    torch.from_numpy(lens).cuda(), torch.from_numpy(starts).cuda(),
                                    torch.from_numpy(np.ascontiguousarray(sh)).cuda(), gsz, mc,
                                    scale, ws, partition_size)
    return out, (starts, shared)


CASES = [
    ("shared_prefix_bs16_cow", dict(batch=6, num_blocks=512)),
    ("shared_prefix_bs16", dict(batch=5, num_blocks=512)),
    ("shared_prefix_bs8", dict(batch=4, num_blocks=1024)),
    ("shared_prefix_bs32_cow", dict(batch=5, num_blocks=256)),
    # Grouped-query heads: the per-sequence pass runs on matrix cores too.
    ("shared_prefix_bs16_cow", dict(batch=5, num_blocks=512, num_q_heads=32, num_kv_heads=4,
                                    dtype="bf16")),
    # No sharing at all: every row stands alone and the cascade is a plain decode.
    ("llama7b", dict(batch=4, num_blocks=1024)),
]


@pytest.mark.parametrize("name,overrides", CASES, ids=[f"{c[0]}-{i}" for i, c in enumerate(CASES)])
@pytest.mark.parametrize("partition_size", [-1, 64])
def test_cascade_matches_oracle(name, overrides, partition_size):
    cfg = W.get_config(name, **overrides)
    print(f"[case] cascade {cfg.name} {overrides} partition {partition_size}", flush=True)
    w = W.make_workload(cfg, device="cuda")
    g = gpu_side.build(w)
    o = oracle_side.build(gpu_side.to_cpu(w), fill=gpu_side.SENTINEL_BITS[cfg.dtype])
    ref = o.decode()
    rows = list(range(w.batch))
    out, (starts, shared) = cascade(g.alloc, rows, w.q[0], g.k_cache, g.v_cache, cfg.scale,
                                    partition_size)
    if cfg.prefix_len:
        assert starts.tolist() == [0, w.batch] and shared[0] > 0
    else:
        assert shared.max() == 0
    err = check(out.double().cpu().numpy(), ref, cfg.dtype, "cascade")
    plain = g.decode(partition_size=partition_size).double().cpu().numpy()
    check(plain, ref, cfg.dtype, "plain decode")
    print(f"  max abs err {err:.3g}; groups {starts.tolist()} shared {shared[:1].tolist()}",
          flush=True)


def test_cascade_two_groups_singleton_and_short_member():
    """Two groups with different prefixes, a row alone, and a group member whose context is
    shorter than the others' shared run."""
    torch.manual_seed(7)
    hq, hkv, d, bs, nblocks = 8, 8, 128, 16, 256
    dt = torch.float16
    a = pkv.PkvAlloc(nblocks, bs, np.random.default_rng(3).permutation(nblocks).astype(np.int32))
    o = oracle.OracleAllocator(nblocks, bs, np.random.default_rng(3).permutation(nblocks))
    kc = torch.empty((nblocks, hkv, bs, d), dtype=dt, device="cuda")
    vc = torch.empty_like(kc)
    gpu_side.fill_bits(kc, "f16", gpu_side.SENTINEL_BITS["f16"])
    gpu_side.fill_bits(vc, "f16", gpu_side.SENTINEL_BITS["f16"])
    kp = oracle.new_pool(nblocks, hkv, bs, d, "f16", gpu_side.SENTINEL_BITS["f16"])
    vp = oracle.new_pool(nblocks, hkv, bs, d, "f16", gpu_side.SENTINEL_BITS["f16"])

    def write(slots, n):
        k = torch.randn((n, hkv, d), dtype=torch.float32, device="cuda").to(dt)
        v = torch.randn((n, hkv, d), dtype=torch.float32, device="cuda").to(dt)
        pkv.pkv_reshape_and_cache(k, v, torch.from_numpy(np.asarray(slots, np.int64)).cuda(), kc, vc)
        oracle.cache_write(kp, oracle.bits_of(k.cpu(), "f16"), slots)
        oracle.cache_write(vp, oracle.bits_of(v.cpu(), "f16"), slots)

    # Prefix A (parent 100: 100 tokens, 6 full blocks + 4) forked to rows 0..2; prefix B
    # (parent 101: 64 tokens) to rows 3..4.
    for parent, n, kids in ((100, 100, [0, 1, 2]), (101, 64, [3, 4])):
        sc = a.pkv_seq_add(parent, n)
        so = o.add(parent, n)
        assert sc.tolist() == so
        write(so, n)
        for kid in kids:
            a.pkv_seq_fork(parent, kid)
            o.fork(parent, kid)
        a.pkv_seq_free(parent)
        o.free_seq(parent)
    sc = a.pkv_seq_add(5, 37)  # alone
    so = o.add(5, 37)
    assert sc.tolist() == so
    write(so, 37)
    # Own tokens: rows 0, 1, 3, 4 grow, copying A's partly filled seventh block on their first
    # write; row 2 keeps the original and stays at 100 tokens, the group's shortest member.
    for row, extra in ((0, 40), (1, 3), (3, 70), (4, 1)):
        for _ in range(extra):
            slots, pairs = a.pkv_seq_append([row])
            so, po = o.append([row])
            assert slots.tolist() == so and pairs.tolist() == [list(p) for p in po]
            if pairs.size:
                pkv.pkv_copy_blocks(kc, vc, torch.from_numpy(pairs).cuda())
                oracle.copy_blocks(kp, po)
                oracle.copy_blocks(vp, po)
            write(so, 1)
    rows = [0, 1, 2, 3, 4, 5]
    starts, shared = a.pkv_prefix_groups(rows)
    assert (starts.tolist(), shared.tolist()) == tuple(o.prefix_groups(rows))
    assert starts.tolist() == [0, 3, 5, 6] and shared.tolist() == [6, 6, 6, 4, 4, 0]
    q = torch.randn((6, hq, d), dtype=torch.float32, device="cuda").to(dt)
    scale = 1.0 / np.sqrt(d)
    out, _ = cascade(a, rows, q, kc, vc, scale)
    mb = max(len(o.tables[r]) for r in rows)
    tab, lens = o.block_tables(rows, mb)
    ref = oracle.decode(oracle.bits_of(q.cpu(), "f16"), kp, vp, tab, lens, scale, "f16")
    err = check(out.double().cpu().numpy(), ref, "f16", "cascade, two groups")
    print(f"  max abs err {err:.3g}", flush=True)


@pytest.mark.parametrize("name,overrides", [
    ("shared_prefix_bs16_cow", dict(batch=6, num_blocks=512)),
    ("shared_prefix_bs16_cow", dict(batch=5, num_blocks=512, num_q_heads=32, num_kv_heads=4,
                                    dtype="bf16")),
])
def test_cascade_launch_bound_and_member_counts(name, overrides):
    """max_group_size only sizes the launch: a bound of 1 (one column tile per group and KV
    head) covers every tile by striding and gives bit-identical output.  The group's shared
    count is its first row's: other members' shared_blocks entries are not read."""
    cfg = W.get_config(name, **overrides)
    w = W.make_workload(cfg, device="cuda")
    g = gpu_side.build(w)
    rows = list(range(w.batch))
    ref, (starts, shared) = cascade(g.alloc, rows, w.q[0], g.k_cache, g.v_cache, cfg.scale)
    assert starts.tolist() == [0, w.batch]
    small, _ = cascade(g.alloc, rows, w.q[0], g.k_cache, g.v_cache, cfg.scale, max_group_size=1)
    assert torch.equal(small, ref)
    big, _ = cascade(g.alloc, rows, w.q[0], g.k_cache, g.v_cache, cfg.scale,
                     max_group_size=4 * w.batch)
    assert torch.equal(big, ref)
    odd = shared.copy()
    odd[1:] = np.arange(1, w.batch) * 1000 - 3  # nonsense in every member but the first
    other, _ = cascade(g.alloc, rows, w.q[0], g.k_cache, g.v_cache, cfg.scale, shared_override=odd)
    assert torch.equal(other, ref)
