"""Paged causal prefill on the GPU against the CPU oracle, on identical seeded inputs.

Bars: block tables, slots and pools bit-exact; outputs within the attention bar of
tests/tolerance.py (5e-3 for fp16/bf16 K/V, widened only where the output type's own
rounding exceeds it).  Pools start filled with a quiet-NaN pattern, so a masked or unused
slot that leaked into an output would show up.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import gpu_side, oracle_side
from tests.tolerance import check

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def both(name, **overrides):
    cfg = W.get_config(name, **overrides)
    print(f"[case] {cfg.name} {overrides}", flush=True)
    w = W.make_workload(cfg, device="cuda")
    g = gpu_side.build(w)
    o = oracle_side.build(gpu_side.to_cpu(w), fill=gpu_side.SENTINEL_BITS[cfg.dtype])
    return w, g, o


def check_all(w, g, o):
    assert [(op, s, [list(p) for p in pr]) for op, s, pr in g.log] == \
        [(op, list(s), [list(p) for p in pr]) for op, s, pr in o.log]
    tg, lg = g.tables()
    to, lo = o.tables()
    assert np.array_equal(tg, to) and np.array_equal(lg, lo)
    dt = w.cfg.dtype
    assert np.array_equal(oracle.bits_of(g.k_cache.cpu(), dt), o.k_pool)
    assert np.array_equal(oracle.bits_of(g.v_cache.cpu(), dt), o.v_pool)
    out = g.prefill().double().cpu().numpy()
    err = check(out, o.prefill(), dt, w.cfg.name)
    print(f"  max abs err {err:.3g}", flush=True)


REDUCED = [
    ("prefill_llama7b", dict(batch=4, lengths=("fixed", (1, 17, 100, 300)), num_blocks=64)),
    ("prefill_chunked_gqa", dict(batch=2, lengths=("fixed", (700, 1500)), num_blocks=160)),
    ("prefill_chunked_gqa", dict(batch=3, lengths=("fixed", (40, 513, 600)),
                                 new_tokens=("fixed", 33), num_blocks=160)),
]


@pytest.mark.parametrize("name,overrides", REDUCED, ids=["fresh", "chunk512", "chunk33"])
def test_prefill_parity(name, overrides):
    check_all(*both(name, **overrides))


SHAPES = []
for dtype in ("f16", "bf16"):
    for d in (64, 128):
        for bs in (8, 16, 32):
            for hq, hkv in ((4, 4), (8, 2), (16, 1), (6, 2)):
                SHAPES.append((dtype, d, bs, hq, hkv))


@pytest.mark.parametrize("dtype,d,bs,hq,hkv", SHAPES)
def test_prefill_shape_sweep(dtype, d, bs, hq, hkv):
    # Ragged new-token counts around the 16-token column tiles, the 32-token wave tiles and
    # the 128-token workgroup tiles, fresh prompts and chunks on top of cached context.
    lengths = (1, 15, 16, 17, 64, 65, 130, 200)
    for new in (("all",), ("fixed", 47)):
        cfg = dict(dtype=dtype, head_dim=d, block_size=bs, num_q_heads=hq, num_kv_heads=hkv,
                   batch=len(lengths), lengths=("fixed", lengths), new_tokens=new,
                   num_blocks=(sum(lengths) // bs + 16) * 2)
        check_all(*both("prefill_llama7b", **cfg))


@pytest.mark.parametrize("factor", [-1.0, 0.0, 3.0])
def test_prefill_any_scale(factor):
    """Negative, zero and large scales (the kernel folds the scale's sign into the query)."""
    for dtype in ("f16", "bf16"):
        w, g, o = both("prefill_chunked_gqa", batch=2, lengths=("fixed", (300, 700)),
                       new_tokens=("fixed", 140), num_blocks=80, dtype=dtype)
        scale = factor * w.cfg.scale
        out = g.prefill(scale=scale).double().cpu().numpy()
        err = check(out, o.prefill(scale=scale), dtype, f"scale {scale}")
        print(f"  {dtype} scale {scale:.4g}: max abs err {err:.3g}", flush=True)


def test_prefill_invalid_table_entries():
    """Out-of-range block ids count as empty blocks, in the chunks before the diagonal (where
    the kernel otherwise skips masking), on the diagonal, and in the first chunk."""
    w, g, o = both("prefill_chunked_gqa", batch=3, lengths=("fixed", (700, 400, 300)),
                   new_tokens=("fixed", 150), num_blocks=120)
    c = w.cfg
    tables, lens = o.tables()
    bad = tables.copy()
    bs = c.block_size
    holes = {0: [3, 40], 1: [0, (400 - 150) // bs + 2], 2: [17]}  # block indices per row
    bad[0, 3], bad[0, 40] = -7, c.num_blocks + 5
    bad[1, 0], bad[1, (400 - 150) // bs + 2] = -1, c.num_blocks
    bad[2, 17] = 1 << 30
    out = g.prefill(tables=bad).double().cpu().numpy()
    q = oracle.to_f64(oracle.bits_of(w.q.cpu(), c.dtype), c.dtype)
    qs = w.query_start
    for b, blks in holes.items():
        n = int(qs[b + 1] - qs[b])
        ctx = int(lens[b])
        kv = [(oracle.to_f64(oracle.gather(o.k_pool, tables[b], ctx, g_), c.dtype),
               oracle.to_f64(oracle.gather(o.v_pool, tables[b], ctx, g_), c.dtype))
              for g_ in range(c.num_kv_heads)]
        for i in range(0, n, 7):
            pos = ctx - n + i
            keep = [t for t in range(pos + 1) if t // bs not in blks]
            for h in range(0, c.num_q_heads, 5):
                k, v = kv[h // c.group]
                r = oracle.attention_contiguous(q[int(qs[b]) + i, h], k[keep], v[keep], c.scale)
                check(out[int(qs[b]) + i, h], r, c.dtype, f"b={b} row {i} h={h}")


def test_prefill_bf16_values_beyond_fp16_range():
    """bf16 kernels stage V as fp16 for the probability product and re-run a workgroup in
    the exact bf16 form when a V value of 2^16 or more made its result non-finite.  Here: a
    huge value in a key every row attends, one in a key only later rows attend (masked for
    the earlier rows, so their 0 * inf must not leak), and one in an unused slot past the
    context (never read)."""
    w, g, o = both("prefill_chunked_gqa", batch=2, lengths=("fixed", (300, 700)),
                   new_tokens=("fixed", 140), num_blocks=80, dtype="bf16")
    c = w.cfg
    bs = c.block_size
    tables, lens = o.tables()

    def put(b, pos, head, d, value):
        blk, off = int(tables[b][pos // bs]), pos % bs
        t = torch.tensor([value], dtype=torch.bfloat16)
        g.v_cache[blk, head, off, d] = t.to(g.v_cache.device)[0]
        o.v_pool[blk, head, off, d] = oracle.bits_of(t, "bf16")[0]

    put(0, 10, 3, 5, 3.0e5)                        # attended by every row of sequence 0
    put(1, 700 - 140 + 20, 0, 100, -2.5e5)         # only rows 20.. of sequence 1 see it
    put(1, 700 + 2, 1, 7, 1.0e6)                   # past the context, inside the last block
    out = g.prefill().double().cpu().numpy()
    err = check(out, o.prefill(), "bf16", "V beyond the fp16 range")
    print(f"  max abs err {err:.3g}", flush=True)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_prefill_tiny_values(dtype):
    """V magnitudes across [2^-33, 2^-12]: below fp16's normal range, where the bf16 kernels'
    fp16 staging of V keeps fewer bits or flushes to zero.  That moves each output by at most
    2^-25 (the outputs are convex combinations of the rows).  On top of it come the fp16
    probabilities (2^-11 relative each), fp32 sums and the output's rounding (2^-9 relative),
    all bounded by 2^-8 times A = sum_t p_t |v_t|, the oracle's attention over |V|.  The bar
    here is 2^-25 + 2^-8 A per element, far tighter than 5e-3 at these magnitudes."""
    cfg = W.get_config("prefill_chunked_gqa", batch=2, lengths=("fixed", (300, 700)),
                       new_tokens=("fixed", 140), num_blocks=80, dtype=dtype)
    w = W.make_workload(cfg, device="cuda")
    # Scale token t's values by 2^-(12 + t % 19): exact in bf16 (and in fp16 down to its
    # subnormal range); the same stored values reach the oracle.
    scale = torch.exp2(-(12 + torch.arange(w.v_tok.shape[0], device="cuda") % 19).float())
    w.v_tok.copy_((w.v_tok.float() * scale[:, None, None]).to(w.v_tok.dtype))
    g = gpu_side.build(w)
    o = oracle_side.build(gpu_side.to_cpu(w), fill=gpu_side.SENTINEL_BITS[dtype])
    out = g.prefill().double().cpu().numpy()
    ref = o.prefill()
    tables, lens = o.tables()
    v_abs = o.v_pool & np.uint16(0x7FFF)  # |v|: the sign bit cleared (fp16 and bf16)
    a = oracle.prefill(oracle.bits_of(o.w.q, dtype), o.k_pool, v_abs, tables, lens,
                       w.query_start, cfg.scale, dtype)
    err = np.abs(out - ref)
    bound = 2.0 ** -25 + 2.0 ** -8 * a
    assert np.all(np.isfinite(out))
    assert np.all(err <= bound), f"max excess {float(np.max(err - bound)):.3g}"
    assert float(np.abs(ref).max()) > 2.0 ** -16  # the outputs are not all below the bound
    print(f"  max abs err {float(err.max()):.3g} with |ref| up to {float(np.abs(ref).max()):.3g}",
          flush=True)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("pattern", ["rising", "sawtooth"])
def test_prefill_reference_moves_many_times(dtype, pattern):
    """Scores that climb along the keys, so that a column's running reference has to move
    again and again during one walk (the kernel moves it only when an fp16 probability
    overflows, i.e. a score climbs about 16 above it in log2 units, or while it is -inf).
    Key t of a sequence is (t' / 512) * (1, .., 1), the query 8 * (1, .., 1): the score of
    key t is 2 t' and its log2-domain exponent 2 t' * scale * log2(e) ~ 0.255 t', about 8
    more per 32-key chunk.  rising: t' = t, so the reference moves every few chunks and
    every earlier key's weight underflows; sawtooth: t' = t mod 160, so the score climbs,
    falls back far below the reference and climbs again."""
    cfg = W.get_config("prefill_llama7b", batch=2, lengths=("fixed", (300, 900)),
                       num_blocks=128, dtype=dtype)
    print(f"[case] reference moves {dtype} {pattern}", flush=True)
    w = W.make_workload(cfg, device="cuda")
    qs = [int(x) for x in w.query_start]
    pos = torch.cat([torch.arange(qs[b + 1] - qs[b]) for b in range(len(qs) - 1)]).to("cuda")
    tp = pos if pattern == "rising" else pos % 160
    w.k_tok.copy_((tp.float() / 512.0)[:, None, None].expand_as(w.k_tok).to(w.k_tok.dtype))
    w.q.fill_(8.0)
    g = gpu_side.build(w)
    o = oracle_side.build(gpu_side.to_cpu(w), fill=gpu_side.SENTINEL_BITS[dtype])
    out = g.prefill().double().cpu().numpy()
    err = check(out, o.prefill(), dtype, f"reference moves, {pattern}")
    print(f"  max abs err {err:.3g}", flush=True)


def test_prefill_matches_decode_kernel_on_the_last_row():
    """The newest row of a prefill and a decode of that sequence read the same keys."""
    w, g, o = both("prefill_chunked_gqa", batch=2, lengths=("fixed", (300, 77)), num_blocks=80)
    out = g.prefill()
    qs = w.query_start
    last = torch.stack([w.q[int(qs[b + 1]) - 1] for b in range(w.batch)])
    dec = g.decode(q=last.contiguous(), partition_size=0)
    for b in range(w.batch):
        check(out[int(qs[b + 1]) - 1].double().cpu().numpy(), dec[b].double().cpu().numpy(),
              w.cfg.dtype, f"b={b}")


@pytest.mark.parametrize("name", ["prefill_llama7b", "prefill_chunked_gqa"])
def test_prefill_full_size_sampled(name):
    cfg = W.get_config(name)
    print(f"[case] full-size {name}", flush=True)
    w = W.make_workload(cfg, device="cuda")
    g = gpu_side.build(w)
    o = oracle_side.OracleState(w, cache=False)
    o.run(W.setup_ops(w))
    o.run(W.step_ops(w))
    for (op_g, s_g, p_g), (op_o, s_o, p_o) in zip(g.log, o.log):
        assert op_g == op_o and s_g == list(s_o) and p_g == [list(p) for p in p_o]
    tg, lg = g.tables()
    to, lo = o.tables()
    assert np.array_equal(tg, to) and np.array_equal(lg, lo)
    out = g.prefill()
    dt = cfg.dtype
    q = oracle.to_f64(oracle.bits_of(w.q.cpu(), dt), dt)
    qs = w.query_start
    rng = np.random.default_rng(0)
    worst = 0.0
    for _ in range(24):
        b = int(rng.integers(w.batch))
        n, ctx = int(w.n_new[b]), int(w.lengths[b])
        i = int(rng.choice([0, n - 1, int(rng.integers(n))]))
        h = int(rng.integers(cfg.num_q_heads))
        pos = ctx - n + i
        k, v = w.token_kv(b, 0, pos + 1)
        g_ = h // cfg.group
        kk = oracle.to_f64(oracle.bits_of(k[:, g_].cpu(), dt), dt)
        vv = oracle.to_f64(oracle.bits_of(v[:, g_].cpu(), dt), dt)
        ref = oracle.attention_contiguous(q[qs[b] + i, h], kk, vv, cfg.scale)
        err = check(out[qs[b] + i, h].double().cpu().numpy(), ref, dt, f"b={b} i={i} h={h}")
        worst = max(worst, err)
    print(f"  worst sampled max abs err {worst:.3g}", flush=True)


@pytest.mark.parametrize("bound", [1, 4, 40])
def test_prefill_loose_query_bound(bound):
    """max_query_len only sizes the launch: a bound above the longest chunk adds row tiles
    (numbered from the end, so the real tiles move to other workgroups) and changes
    nothing."""
    w, g, o = both("prefill_chunked_gqa", batch=3, lengths=("fixed", (40, 513, 600)),
                   new_tokens=("fixed", 33), num_blocks=160)
    ref = o.prefill()
    mq = int(np.max(np.diff(w.query_start)))
    out = g.prefill(max_query_len=bound * mq + (bound > 1)).double().cpu().numpy()
    check(out, ref, w.cfg.dtype, f"max_query_len {bound} x")
