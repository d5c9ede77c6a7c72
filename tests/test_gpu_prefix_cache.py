"""Automatic prefix caching end to end on the GPU (needs an MI355X).

Full prompt blocks are keyed by their tokens and everything before them; a
new sequence with the same beginning reuses those blocks and writes only the
rest of its prompt, which saves prompt processing and leaves decode
unchanged [F55 §后来的做法].  Each position's K/V here is a function of the
whole token prefix up to it (as a model's would be), so a reused block is
right only if the prefix matched.  Decode over the cached pool must be
bit-identical to decode over a pool where every sequence wrote its whole
prompt into blocks of its own.
"""
import zlib

import numpy as np
import pytest
import torch

from paged_kv_cache_375_amd import api

pytestmark = pytest.mark.gpu

CASES = [("f16", 16, 8, 2, 128), ("e4m3", 16, 8, 8, 128), ("f32", 4, 2, 2, 64)]


def _rows(tokens, hkv, d, act):
    """K and V rows [n][hkv][d]: position p's values depend on tokens[:p + 1] only."""
    k = np.empty((len(tokens), hkv, d), np.float32)
    v = np.empty_like(k)
    for p in range(len(tokens)):
        g = np.random.default_rng(zlib.crc32(np.asarray(tokens[: p + 1], np.int32).tobytes()))
        k[p] = g.standard_normal((hkv, d))
        v[p] = g.standard_normal((hkv, d))
    return torch.from_numpy(k).to(act).cuda(), torch.from_numpy(v).to(act).cuda()


def _write(cache, alloc, seq, tokens, start, max_blocks, act):
    k, v = _rows(tokens, cache.num_kv_heads, cache.head_dim, act)
    tables, _ = alloc.export([seq], max_blocks)
    n = len(tokens) - start
    i64 = lambda x: torch.tensor([x], dtype=torch.int64).cuda()
    i32 = lambda x: torch.tensor([x], dtype=torch.int32).cuda()
    api.kv_write_prompt(cache, k, v, i64(start), i32(start), i32(n), torch.from_numpy(tables).cuda(), max(n, 1))
    return n


@pytest.mark.parametrize("case", CASES, ids=lambda c: "{}_bs{}_q{}_kv{}_d{}".format(*c))
def test_cached_prompts_decode_bit_identical(case):
    kv, bs, hq, hkv, d = case
    print(f"[prefix-cache] {case}", flush=True)
    act = torch.float32 if kv == "f32" else torch.float16
    rng = np.random.default_rng(21)
    system = rng.integers(0, 50, 300).tolist()
    prompts = [system + rng.integers(0, 50, 77).tolist(),        # writes everything
               system[:200] + rng.integers(0, 50, 333).tolist(),  # shares 200 tokens' full blocks
               system + rng.integers(0, 50, 9).tolist(),          # shares the 300-token system prompt
               rng.integers(0, 50, 41).tolist() + system]         # the same tokens later: nothing shared
    need = [-(-len(p) // bs) for p in prompts]
    max_blocks, max_ctx = max(need), max(len(p) for p in prompts)
    nb = sum(need) + 8
    scale = dict(k_scale=0.02, v_scale=0.02, k_inv_scale=50.0, v_inv_scale=50.0) if kv == "e4m3" else {}
    perm = np.random.default_rng(5).permutation(nb)

    cached_alloc = api.Allocator(nb, bs, perm)
    cached_pool = api.KVCache(nb, bs, hkv, d, kv, "cuda", **scale)
    written = []
    for s, p in enumerate(prompts):
        start = cached_alloc.allocate_cached(s, p)
        written.append(_write(cached_pool, cached_alloc, s, p, start, max_blocks, act))
    assert written[0] == len(prompts[0])
    assert written[1] == len(prompts[1]) - 200 // bs * bs
    assert written[2] == len(prompts[2]) - 300 // bs * bs
    assert written[3] == len(prompts[3])
    assert cached_alloc.table(2)[: 300 // bs] == cached_alloc.table(0)[: 300 // bs]

    plain_alloc = api.Allocator(nb, bs, perm[::-1].copy())
    plain_pool = api.KVCache(nb, bs, hkv, d, kv, "cuda", **scale)
    for s, p in enumerate(prompts):
        plain_alloc.allocate(s, len(p))
        _write(plain_pool, plain_alloc, s, p, 0, max_blocks, act)

    q = torch.randn(len(prompts), hq, d, generator=torch.Generator().manual_seed(3)).to(act).cuda()
    outs = []
    for alloc, pool in ((cached_alloc, cached_pool), (plain_alloc, plain_pool)):
        t, c = alloc.export(list(range(len(prompts))), max_blocks)
        outs.append(api.decode(pool, q, torch.from_numpy(t).cuda(), torch.from_numpy(c).cuda(), max_ctx,
                               d ** -0.5))
    torch.cuda.synchronize()
    assert torch.isfinite(outs[0].float()).all()
    assert torch.equal(outs[0], outs[1])
    print(f"[prefix-cache] {case}: wrote {sum(written)} of {sum(map(len, prompts))} prompt rows, "
          f"decode bit-identical", flush=True)
