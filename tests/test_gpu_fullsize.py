"""Full-size workloads in the launch configuration the benchmark times (automatic 512-token
partitions), checked against the oracle where it can compute outputs one by one:
  * the allocator's whole request schedule (every slot, every copy-on-write pair, every
    table) replayed on the oracle allocator: bit-exact;
  * sampled cache rows read back from the pools: bit-exact against the token they hold;
  * sampled (sequence, head) outputs against the plain fp64 definition over that sequence's
    contiguous K/V: within 5e-3 (fp16/bf16 K/V); for the shared-prefix workloads also the
    cascade decode's.
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

FULL = ["llama7b", "llama13b", "gqa_long", "shared_prefix_bs8_cow", "shared_prefix_bs16_cow",
        "shared_prefix_bs32_cow", "shared_prefix_bs8", "shared_prefix_bs16", "shared_prefix_bs32"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    cfg = W.get_config(name, steps=1)
    print(f"[case] full-size {name}", flush=True)
    w = W.make_workload(cfg, device="cuda")
    g = gpu_side.build(w)
    o = oracle_side.OracleState(w, cache=False)
    o.run(W.setup_ops(w))
    o.run(W.step_ops(w))
    assert len(g.log) == len(o.log)
    for (op_g, s_g, p_g), (op_o, s_o, p_o) in zip(g.log, o.log):
        assert op_g == op_o and s_g == list(s_o) and p_g == [list(p) for p in p_o]
    tg, lg = g.tables()
    to, lo = o.tables()
    assert np.array_equal(tg, to) and np.array_equal(lg, lo)
    assert np.array_equal(lg, w.lengths)

    rng = np.random.default_rng(0)
    bs, dt = cfg.block_size, cfg.dtype
    # Sampled cache rows: token t of sequence b sits at slot table[t // bs] * bs + t % bs.
    for _ in range(64):
        b = int(rng.integers(w.batch))
        t = int(rng.integers(int(lo[b])))
        blk = int(to[b][t // bs])
        k, v = w.token_kv(b, t, t + 1)
        assert torch.equal(g.k_cache[blk, :, t % bs, :], k[0])
        assert torch.equal(g.v_cache[blk, :, t % bs, :], v[0])

    # The automatic split the benchmark times; the long-context GQA workload also in the
    # 512-token partitions its description names.
    outs = {p: g.decode(partition_size=p) for p in ([-1, 512] if name == "gqa_long" else [-1])}
    if cfg.prefix_len:  # the shared-prefix workloads are also timed as a cascade decode
        from tests.test_gpu_cascade import cascade
        outs["cascade"], (starts, shared) = cascade(g.alloc, list(range(w.batch)), w.q[0],
                                                    g.k_cache, g.v_cache, cfg.scale)
        assert starts.tolist() == [0, w.batch] and int(shared[0]) == cfg.prefix_len // bs
    order = np.argsort(w.lengths)
    picks = {(int(order[0]), 0), (int(order[-1]), cfg.num_q_heads - 1)}
    while len(picks) < 24:
        picks.add((int(rng.integers(w.batch)), int(rng.integers(cfg.num_q_heads))))
    q = oracle.to_f64(oracle.bits_of(w.q[0].cpu(), dt), dt)
    worst = 0.0
    for b, h in sorted(picks):
        n = int(w.lengths[b])
        k, v = w.token_kv(b, 0, n)
        g_ = h // cfg.group
        kk = oracle.to_f64(oracle.bits_of(k[:, g_].cpu(), dt), dt)
        vv = oracle.to_f64(oracle.bits_of(v[:, g_].cpu(), dt), dt)
        ref = oracle.attention_contiguous(q[b, h], kk, vv, cfg.scale)
        for p, out in outs.items():
            assert bool(torch.isfinite(out[b, h]).all())
            err = check(out[b, h].double().cpu().numpy(), ref, dt, f"p={p} b={b} h={h} ctx={n}")
            worst = max(worst, err)
    print(f"  worst sampled max abs err {worst:.3g}", flush=True)
