"""Preemption by swapping on the GPU (needs an MI355X).

When blocks run out, the latest arrival gives up all of its blocks and its
K/V move to host memory; when it resumes, it takes fresh blocks and the K/V
move back [F55 §放不下的时候].  A correct round trip is invisible to
attention: the resumed sequence's output must be bit-identical to the one
before preemption, even though a sequence that ran in between reused (and
overwrote) the very blocks it gave up.  The host copy must hold each block's
bytes exactly.
"""
import numpy as np
import pytest
import torch

from paged_kv_cache_375_amd import api
from tests.gpu_helpers import pool_bytes

pytestmark = pytest.mark.gpu

# (pool dtype, block size, KV heads, head_dim)
CASES = [("f16", 16, 8, 128), ("f32", 4, 2, 64), ("e4m3", 1, 4, 32), ("e4m3", 16, 1, 128)]


def _prompt(cache, alloc, seq, rows, act, max_blocks, gen):
    """Write a random prompt of `rows` tokens for seq into its blocks."""
    k = torch.randn(rows, cache.num_kv_heads, cache.head_dim, generator=gen).to(act).cuda()
    v = torch.randn(rows, cache.num_kv_heads, cache.head_dim, generator=gen).to(act).cuda()
    tables, _ = alloc.export([seq], max_blocks)
    i64 = lambda x: torch.tensor([x], dtype=torch.int64).cuda()
    i32 = lambda x: torch.tensor([x], dtype=torch.int32).cuda()
    api.kv_write_prompt(cache, k, v, i64(0), i32(0), i32(rows), torch.from_numpy(tables).cuda(), rows)


def _decode(cache, alloc, q, seqs, max_blocks, max_ctx):
    tables, ctx = alloc.export(seqs, max_blocks)
    return api.decode(cache, q, torch.from_numpy(tables).cuda(), torch.from_numpy(ctx).cuda(), max_ctx,
                      q.shape[-1] ** -0.5).clone()


@pytest.mark.parametrize("case", CASES, ids=lambda c: "{}_bs{}_kv{}_d{}".format(*c))
def test_swap_round_trip_bit_exact_and_decode_unchanged(case):
    kv, bs, hkv, d = case
    print(f"[swap] {case}", flush=True)
    act = torch.float32 if kv == "f32" else torch.float16
    gen = torch.Generator().manual_seed(100 + CASES.index(case))
    lens = [700, 333]                      # sequence 1 arrives last
    need = [-(-n // bs) for n in lens]
    nb = sum(need) + 1                     # tight: whoever runs next must reuse sequence 1's blocks
    max_blocks, max_ctx = max(need), max(lens)
    alloc = api.Allocator(nb, bs, np.random.default_rng(1).permutation(nb))
    scale = dict(k_scale=0.05, v_scale=0.04, k_inv_scale=20.0, v_inv_scale=25.0) if kv == "e4m3" else {}
    cache = api.KVCache(nb, bs, hkv, d, kv, "cuda", **scale)
    for s, n in enumerate(lens):
        alloc.allocate(s, n)
        _prompt(cache, alloc, s, n, act, max_blocks, gen)
    q = torch.randn(2, 2 * hkv, d, generator=gen).to(act).cuda()
    before = _decode(cache, alloc, q, [0, 1], max_blocks, max_ctx)

    victim = alloc.latest_arrival()
    assert victim == 1
    out_ids = alloc.swap_out(victim)
    n = len(out_ids)
    host_k = torch.empty((n, hkv, bs, d), dtype=cache.k.dtype).pin_memory()
    host_v = torch.empty_like(host_k).pin_memory()
    api.swap_blocks(cache, host_k, host_v, torch.tensor(out_ids, dtype=torch.int32).cuda(), "out")
    torch.cuda.synchronize()
    ids = np.array(out_ids)
    assert np.array_equal(host_k.numpy().view(np.uint8), pool_bytes(cache.k)[ids])
    assert np.array_equal(host_v.numpy().view(np.uint8), pool_bytes(cache.v)[ids])

    # another sequence runs in the freed blocks and overwrites them
    intruder_len = alloc.num_free() * bs
    alloc.allocate(2, intruder_len)
    assert set(out_ids) <= set(alloc.table(2))
    _prompt(cache, alloc, 2, intruder_len, act, -(-intruder_len // bs), gen)
    torch.cuda.synchronize()
    assert not np.array_equal(pool_bytes(cache.k)[ids], host_k.numpy().view(np.uint8))
    alloc.free_seq(2)

    in_ids = alloc.swap_in(victim)
    assert len(in_ids) == n and in_ids != out_ids  # fresh blocks, placed elsewhere
    api.swap_blocks(cache, host_k, host_v, torch.tensor(in_ids, dtype=torch.int32).cuda(), "in")
    after = _decode(cache, alloc, q, [0, 1], max_blocks, max_ctx)
    torch.cuda.synchronize()
    assert torch.equal(before, after)
    print(f"[swap] {case}: {n} blocks out and back, decode bit-identical", flush=True)


def test_swap_skips_out_of_range_ids():
    cache = api.KVCache(8, 4, 2, 32, "f16", "cuda")
    cache.k.copy_(torch.randn_like(cache.k, dtype=torch.float32).half())
    cache.v.copy_(torch.randn_like(cache.v, dtype=torch.float32).half())
    keep_k, keep_v = cache.k.clone(), cache.v.clone()
    host_k = torch.full((3, 2, 4, 32), 7.0, dtype=torch.float16).pin_memory()
    host_v = torch.full((3, 2, 4, 32), 9.0, dtype=torch.float16).pin_memory()
    ids = torch.tensor([-1, 5, 8], dtype=torch.int32).cuda()
    api.swap_blocks(cache, host_k, host_v, ids, "in")
    torch.cuda.synchronize()
    assert torch.equal(cache.k[5], host_k[1].cuda()) and torch.equal(cache.v[5], host_v[1].cuda())
    others = [b for b in range(8) if b != 5]
    assert torch.equal(cache.k[others], keep_k[others]) and torch.equal(cache.v[others], keep_v[others])
    api.swap_blocks(cache, host_k, host_v, ids, "out")
    torch.cuda.synchronize()
    assert torch.equal(host_k[0], torch.full((2, 4, 32), 7.0, dtype=torch.float16))  # skipped entries untouched
    assert torch.equal(host_k[1].cuda(), cache.k[5])
