"""Cases of decode attention whose result the mathematics fixes exactly ("PagedAttention 与
vLLM 推理加速", §1: the new token's output is the softmax-weighted sum of the values of every
cached token), checked on the GPU against the closed form rather than the oracle:
  * a context of one token: the weight is 1, so the output is that token's value row, bit
    for bit (the stored type holds it exactly);
  * a zero query, or keys that are all equal: every score is the same, the weights are
    uniform, and the output is the mean of the value rows, within the parity bar.
Each runs on the VALU kernels (every element type, one query head per KV head) and on the
matrix-core kernels (grouped-query heads, fp16 and bf16), unsplit and split into short
partitions so that the partition merge takes part.
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests import gpu_side
from tests.tolerance import check

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

# (base workload, overrides): VALU instances first, then matrix-core (GQA) instances.
PATHS = [
    ("tiny", dict(dtype="f32")),
    ("tiny", dict(dtype="f16", head_dim=64, block_size=8, num_q_heads=4, num_kv_heads=4)),
    ("llama7b", dict(num_q_heads=4, num_kv_heads=4)),                   # bf16, D=128, bs=16
    ("gqa_long", dict()),                                               # bf16, group 8
    ("gqa_long", dict(dtype="f16", block_size=32, num_q_heads=16, num_kv_heads=2)),
]
PARTS = [-1, 0, 32]


def ids(p):
    return f"{p[0]}-{p[1].get('dtype', W.get_config(p[0]).dtype)}-hq{p[1].get('num_q_heads', W.get_config(p[0]).num_q_heads)}"


def build(name, ov, lengths):
    cfg = W.get_config(name, batch=len(lengths), lengths=("fixed", tuple(lengths)),
                       num_blocks=sum(-(-n // 4) for n in lengths) + 64, steps=1, **ov)
    print(f"[case] {name} {ov} lengths {lengths}", flush=True)
    return cfg, W.make_workload(cfg, device="cuda")


def values_f64(w, b, g):
    _, v = w.token_kv(b, 0, int(w.lengths[b]))
    return v[:, g].double().cpu().numpy()


@pytest.mark.parametrize("path", PATHS, ids=[ids(p) for p in PATHS])
def test_one_token_context_returns_its_value_row(path):
    name, ov = path
    cfg, w = build(name, ov, [1, 1, 1])
    g = gpu_side.build(w)
    for p in PARTS:
        out = g.decode(partition_size=p)
        for b in range(w.batch):
            _, v = w.token_kv(b, 0, 1)
            for h in range(cfg.num_q_heads):
                assert torch.equal(out[b, h], v[0, h // cfg.group]), (p, b, h)


@pytest.mark.parametrize("path", PATHS, ids=[ids(p) for p in PATHS])
def test_zero_query_gives_the_mean_of_the_values(path):
    name, ov = path
    cfg, w = build(name, ov, [1, 2, 17, 300])
    g = gpu_side.build(w)
    q0 = torch.zeros_like(w.q[0])
    for p in PARTS:
        out = g.decode(partition_size=p, q=q0).double().cpu().numpy()
        for b in range(w.batch):
            for kh in range(cfg.num_kv_heads):
                mean = values_f64(w, b, kh).mean(axis=0)
                for h in range(kh * cfg.group, (kh + 1) * cfg.group):
                    check(out[b, h], mean, cfg.dtype, f"q=0 p={p} b={b} h={h}")


@pytest.mark.parametrize("path", PATHS, ids=[ids(p) for p in PATHS])
def test_equal_keys_give_the_mean_of_the_values(path):
    name, ov = path
    cfg, w = build(name, ov, [2, 31, 300, 5])
    # Every key row of every sequence and head becomes the first token's key of head 0.
    row = w.k_tok[0, 0].clone()
    w.k_tok[:] = row
    g = gpu_side.build(w)
    for p in PARTS:
        out = g.decode(partition_size=p).double().cpu().numpy()
        for b in range(w.batch):
            for kh in range(cfg.num_kv_heads):
                mean = values_f64(w, b, kh).mean(axis=0)
                for h in range(kh * cfg.group, (kh + 1) * cfg.group):
                    check(out[b, h], mean, cfg.dtype, f"equal keys p={p} b={b} h={h}")
