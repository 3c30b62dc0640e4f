"""The fused cache write with device-side table upkeep (``pkv_append_and_cache``) called
directly, against the oracle's cache write.

Every case writes n new tokens' K/V rows through their slots into pools that start filled
with a quiet-NaN pattern, so a stray or a missed write shows.  Slots are distinct and include
-1 (skipped) and one past the pool (skipped).  Bars, all bit-exact:
  * both pools against ``oracle.cache_write`` on the same rows and slots;
  * with tables: entry ``pos // block_size`` of the token's row holds ``slot // block_size``
    and the row's length is ``pos + 1``, for every token whose slot is inside the pool;
    nothing else in the tables changes.
Head counts and sizes are chosen so that a workgroup's 256 threads cover the rows of one
token in fewer than, exactly and more than four 16-byte vectors each.  Slots, rows and
positions are given both as device tensors and as pinned host tensors, which the kernel
reads in place (the form the timed decode step uses).
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_359_amd as pkv
from tests import gpu_side

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

CASES = [
    # dtype, Hkv, D, block_size, tokens, blocks; 16-byte vectors per token (K or V):
    ("bf16", 8, 64, 16, 37, 64),      # 64: a quarter of the threads
    ("f16", 40, 128, 16, 53, 256),    # 640: the headline's LLaMA-13B heads
    ("f16", 64, 128, 32, 29, 64),     # 1024: exactly four per thread
    ("f32", 40, 128, 8, 41, 128),     # 1280: four per thread, then a fifth for some
]


@pytest.mark.parametrize("tables", [True, False], ids=["tables", "cache_only"])
@pytest.mark.parametrize("host", [True, False], ids=["pinned", "device"])
@pytest.mark.parametrize("dtype,hkv,d,bs,n,nblk", CASES,
                         ids=[f"{c[0]}_h{c[1]}_d{c[2]}_bs{c[3]}" for c in CASES])
def test_append_and_cache_matches_oracle(dtype, hkv, d, bs, n, nblk, host, tables):
    print(f"[case] append {dtype} Hkv={hkv} D={d} bs={bs} n={n} host={host} tables={tables}",
          flush=True)
    rng = np.random.default_rng(20 + n)
    num_slots = nblk * bs
    slots = rng.choice(num_slots, size=n, replace=False).astype(np.int64)
    slots[3] = -1
    slots[7] = num_slots  # one past the pool
    rows = rng.permutation(n).astype(np.int32)  # one token per row, rows in any order
    max_blocks = 4
    pos = rng.integers(0, max_blocks * bs, size=n).astype(np.int32)

    dev = "cuda"
    key = torch.randn(n, hkv, d, device=dev).to(TORCH[dtype])
    value = torch.randn(n, hkv, d, device=dev).to(TORCH[dtype])
    k_cache = torch.empty(nblk, hkv, bs, d, dtype=TORCH[dtype], device=dev)
    v_cache = torch.empty_like(k_cache)
    gpu_side.fill_bits(k_cache, dtype, gpu_side.SENTINEL_BITS[dtype])
    gpu_side.fill_bits(v_cache, dtype, gpu_side.SENTINEL_BITS[dtype])
    tbl0 = rng.integers(-1, nblk, size=(n, max_blocks)).astype(np.int32)
    lens0 = rng.integers(0, max_blocks * bs, size=n).astype(np.int32)
    block_tables = torch.from_numpy(tbl0).to(dev)
    context_lens = torch.from_numpy(lens0).to(dev)

    def put(a):
        t = torch.from_numpy(a)
        return t.pin_memory() if host else t.to(dev)

    s_t, r_t, p_t = put(slots), put(rows), put(pos)
    if tables:
        pkv.pkv_append_and_cache(key, value, s_t, k_cache, v_cache, block_tables, context_lens,
                                 p_t, r_t)
    else:
        pkv.pkv_append_and_cache(key, value, s_t, k_cache, v_cache)
    torch.cuda.synchronize()

    for new, pool in ((key, k_cache), (value, v_cache)):
        ref = oracle.new_pool(nblk, hkv, bs, d, dtype, fill=gpu_side.SENTINEL_BITS[dtype])
        keep = slots < num_slots
        oracle.cache_write(ref, oracle.bits_of(new.cpu(), dtype)[keep], slots[keep])
        assert np.array_equal(oracle.bits_of(pool.cpu(), dtype), ref)

    tbl, lens = tbl0.copy(), lens0.copy()
    if tables:
        for s, r, p in zip(slots, rows, pos):
            if 0 <= s < num_slots:
                tbl[r, p // bs] = s // bs
                lens[r] = p + 1
    assert np.array_equal(block_tables.cpu().numpy(), tbl)
    assert np.array_equal(context_lens.cpu().numpy(), lens)
