"""Parity of the grouped-query (matrix-core) decode kernel and of the full
workloads against the CPU reference (needs an MI355X).

Small cases cover every head-tile count the kernel is built for, query
groups split over several workgroups, partial head tiles, every head_dim,
FP8 pools and block sizes from 1 to 64; each spans several 512-token
partitions with a ragged last chunk.  The full workloads run at their real
sizes, in the launch the benchmark times, and every output element is
checked against the reference (its decode spread over host threads)."""
import numpy as np
import pytest
import torch

from paged_kv_cache_375_amd.workloads import WORKLOADS, Workload
from tests.gpu_helpers import TOL, build_pair, full_size_check, out_f64, pool_bytes

pytestmark = pytest.mark.gpu

# (q heads, kv heads, head_dim, pool dtype, block size)
GROUP_CASES = [
    (16, 8, 128, "f16", 16),   # G 2
    (64, 8, 128, "f16", 16),   # G 8, the Llama-2-70B layer's grouping
    (32, 2, 128, "f16", 16),   # G 16: one full head tile
    (68, 2, 128, "f16", 16),   # G 34: three tiles over two workgroups per KV head
    (71, 1, 64, "f16", 16),    # G 71: five tiles, the Falcon-7B layer's grouping
    (40, 1, 64, "f16", 32),    # G 40: three tiles
    (24, 1, 32, "f16", 4),     # G 24, head_dim 32, small blocks
    (64, 4, 64, "f16", 1),     # G 16, one token per block
    (64, 8, 128, "f16", 64),   # G 8, 64-token blocks
    (64, 8, 128, "e4m3", 16),  # FP8 pool, head_dim 128
    (40, 4, 64, "e4m3", 8),    # FP8 pool, head_dim 64
    (12, 3, 32, "e4m3", 16),   # FP8 pool, head_dim 32 (8-byte K loads)
    # many head tiles per KV head, more pool dtypes and head sizes
    (71, 1, 64, "e4m3", 16),   # FP8 pool, five tiles
    (80, 2, 128, "e4m3", 16),  # FP8 pool, G 40, head_dim 128: three tiles
    (64, 1, 128, "f16", 64),   # G 64, head_dim 128: four tiles, 64-token blocks
]


def _wl(hq, hkv, d, kv, bs):
    return Workload(f"group_{hq}x{hkv}x{d}_{kv}_bs{bs}", hq, hkv, d, bs, 4, 1, 1300, kv=kv)


@pytest.mark.parametrize("fused", [True, False], ids=["decode_step", "append+decode"])
@pytest.mark.parametrize("case", GROUP_CASES, ids=lambda c: "q{}_kv{}_d{}_{}_bs{}".format(*c))
def test_group_kernel_parity(case, fused):
    wl = _wl(*case)
    print(f"[group] {wl} fused={fused}", flush=True)
    dr, gpu, ref = build_pair(wl)
    out = out_f64(gpu.run(fused=fused))
    ref.append()
    assert np.array_equal(pool_bytes(gpu.cache.k), ref.k.view(np.uint8))
    assert np.array_equal(pool_bytes(gpu.cache.v), ref.v.view(np.uint8))
    want = ref.decode()
    err = float(np.max(np.abs(out - want)))
    print(f"[group] {wl.name}: max abs err {err:.3e} (bound {TOL[wl.kv]})", flush=True)
    assert np.all(np.isfinite(out))
    assert err <= TOL[wl.kv]
    out2 = out_f64(gpu.run(fused=fused))
    assert np.array_equal(out, out2)  # deterministic, counters left at zero


def test_group_kernel_long_partitions():
    """64 sequences x 8 KV heads fill the GPU's resident workgroups in one
    round only with partitions longer than 512 tokens, so the launch picks
    longer ones; contexts are short and ragged."""
    wl = Workload("group_64x8_long_part", 64, 8, 128, 16, 64, 1, 1300)
    print(f"[group] {wl}", flush=True)
    dr, gpu, ref = build_pair(wl)
    out = out_f64(gpu.run())
    ref.append()
    assert np.array_equal(pool_bytes(gpu.cache.k), ref.k.view(np.uint8))
    assert np.array_equal(pool_bytes(gpu.cache.v), ref.v.view(np.uint8))
    err = float(np.max(np.abs(out - ref.decode())))
    print(f"[group] {wl.name}: max abs err {err:.3e}", flush=True)
    assert err <= TOL["f16"]


# Launches with so many (KV head, query group, sequence) units that eight-wave
# workgroups (one per CU, at most two per CU at any register count) cannot
# run them in one round, so the launcher takes four-wave workgroups; with at
# least 2,048 units even those need several rounds, so partitions are 512
# tokens and longer contexts merge in the launch.
# (q heads, kv heads, head_dim, pool dtype, block size, sequences)
FOUR_WAVE_CASES = [
    (16, 8, 128, "f16", 16, 256),    # G 2, head_dim 128
    (64, 32, 64, "f16", 16, 64),     # G 2, head_dim 64
    (48, 16, 32, "f16", 4, 128),     # G 3, head_dim 32, 4-token blocks (per-row addressing)
    (64, 16, 128, "e4m3", 16, 128),  # FP8 pool, head_dim 128
    (40, 8, 64, "e4m3", 8, 256),     # FP8 pool, head_dim 64, 8-token blocks
    (68, 2, 128, "f16", 16, 512),    # G 34: two tiles over two workgroups per KV head
    (71, 1, 64, "f16", 16, 2048),    # G 71: five tiles
]


@pytest.mark.parametrize("case", FOUR_WAVE_CASES, ids=lambda c: "q{}_kv{}_d{}_{}_bs{}_B{}".format(*c))
def test_group_kernel_four_wave_launches(case):
    hq, hkv, d, kv, bs, b = case
    tiles = -(-(hq // hkv) // 16)               # 16-head tiles per KV head
    groups = -(-tiles // (2 if d >= 128 else 5))  # workgroups per KV head (2 or 5 tiles each at most)
    assert hkv * groups * b >= 2048
    wl = Workload(f"group4w_{hq}x{hkv}x{d}_{kv}_bs{bs}_B{b}", hq, hkv, d, bs, b, 1, 700, kv=kv)
    print(f"[group4w] {wl}", flush=True)
    dr, gpu, ref = build_pair(wl)
    out = out_f64(gpu.run())
    ref.append()
    assert np.array_equal(pool_bytes(gpu.cache.k), ref.k.view(np.uint8))
    assert np.array_equal(pool_bytes(gpu.cache.v), ref.v.view(np.uint8))
    want = ref.decode_threaded()
    err = float(np.max(np.abs(out - want)))
    print(f"[group4w] {wl.name}: max abs err {err:.3e} (bound {TOL[wl.kv]})", flush=True)
    assert np.all(np.isfinite(out))
    assert err <= TOL[wl.kv]


def test_group_kernel_placement_invariance_bit_exact():
    wl = _wl(64, 8, 128, "f16", 16)
    dr, gpu, ref = build_pair(wl)
    out = gpu.run().clone()
    from paged_kv_cache_375_amd import api
    perm = torch.randperm(dr.num_blocks, generator=torch.Generator().manual_seed(3)).cuda()
    k2, v2 = torch.empty_like(gpu.cache.k), torch.empty_like(gpu.cache.v)
    k2[perm] = gpu.cache.k
    v2[perm] = gpu.cache.v
    t = gpu.tables.long()
    tables2 = torch.where(t >= 0, perm[t.clamp(min=0)], t).to(torch.int32).contiguous()
    out2 = api.decode(gpu.cache.with_pools(k2, v2), gpu.q, tables2, gpu.ctx, gpu.max_ctx, gpu.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


@pytest.mark.parametrize("hq,hkv,d", [(64, 8, 128), (71, 1, 64)], ids=["gqa", "mqa"])
def test_group_kernel_special_cases(hq, hkv, d):
    from paged_kv_cache_375_amd import api
    G = hq // hkv
    wl = Workload("group_ctx1", hq, hkv, d, 16, 4, 1, 1)
    dr, gpu, ref = build_pair(wl)
    out = gpu.run()
    torch.cuda.synchronize()
    # one token: its weight is exactly one, the output is the appended V
    assert torch.equal(out, gpu.v_new.repeat_interleave(G, dim=1))
    wl = Workload("group_bad", hq, hkv, d, 16, 3, 300, 1100)
    dr, gpu, ref = build_pair(wl)
    gpu.run()
    bad = gpu.tables.clone()
    bad[1, 0] = dr.num_blocks + 3
    outb = api.decode(gpu.cache, gpu.q, bad, gpu.ctx, gpu.max_ctx, gpu.sm_scale)
    ctx0 = torch.zeros_like(gpu.ctx)
    out0 = api.decode(gpu.cache, gpu.q, gpu.tables, ctx0, gpu.max_ctx, gpu.sm_scale)
    torch.cuda.synchronize()
    assert torch.isnan(outb[1]).all()
    assert not torch.isnan(outb[0]).any() and not torch.isnan(outb[2]).any()
    assert torch.count_nonzero(out0) == 0


# opt13b_fp8_prefix505: the 505-token prefix ends inside a block, so every
# sequence's first write copies that shared block first (64 copies)
FULL = ["opt13b", "llama70b_gqa", "falcon7b_mqa", "opt13b_fp8_prefix", "opt13b_fp8_prefix505", "llama70b_gqa_tp8",
        "opt13b_tp8"]


@pytest.mark.parametrize("name", FULL)
def test_full_workload_parity(name):
    """The real sizes in the benchmark's launch (append + decode fused,
    pa_decode_step): the whole pool after the step is bit-exact and every
    output element meets the bound against the reference."""
    wl = WORKLOADS[name]
    print(f"[full] {name}: building", flush=True)
    dr, gpu, ref = build_pair(wl)
    out = out_f64(gpu.run())
    ref.append()
    print(f"[full] {name}: comparing pools", flush=True)
    assert np.array_equal(pool_bytes(gpu.cache.k), ref.k.view(np.uint8))
    assert np.array_equal(pool_bytes(gpu.cache.v), ref.v.view(np.uint8))
    full_size_check(name, wl, out, ref, dr)


@pytest.mark.parametrize("bs", [1, 2, 4, 8, 32, 64])
def test_full_mqa_block_size_sweep(bs):
    """The Falcon-7B MQA layer at its real size at every other block size of
    the sweep (16 is the workload itself, above): the same lengths and K/V
    values, placement re-drawn.  Blocks below 16 tokens take the grouped
    kernel's per-row addressing.  Pool bit-exact, every output element
    within the bound."""
    wl = WORKLOADS["falcon7b_mqa"].with_block_size(bs)
    print(f"[full] {wl.name}: building", flush=True)
    dr, gpu, ref = build_pair(wl)
    out = out_f64(gpu.run())
    ref.append()
    assert np.array_equal(pool_bytes(gpu.cache.k), ref.k.view(np.uint8))
    assert np.array_equal(pool_bytes(gpu.cache.v), ref.v.view(np.uint8))
    full_size_check(wl.name, wl, out, ref, dr)


@pytest.mark.parametrize("scale", [-0.0883883, 0.0, 0.35], ids=["negative", "zero", "large"])
@pytest.mark.parametrize("case", [(71, 1, 64, "f16", 16), (64, 8, 128, "e4m3", 16), (16, 16, 128, "f16", 16)],
                         ids=["mqa_grouped", "gqa_fp8_grouped", "mha_per_head"])
def test_any_finite_scale(case, scale):
    """The score scale may be any finite number.  The grouped kernel keeps
    scores unscaled until the exponent and folds a negative scale into q; a
    zero scale gives every token the same weight (the mean of V), masked
    tokens still none; a large one makes the weights nearly one-hot."""
    wl = _wl(*case)
    print(f"[group] {wl} scale={scale}", flush=True)
    dr, gpu, ref = build_pair(wl)
    gpu.sm_scale = ref.sm_scale = float(np.float32(scale))
    out = out_f64(gpu.run())
    ref.append()
    err = float(np.max(np.abs(out - ref.decode())))
    print(f"[group] {wl.name} scale {scale}: max abs err {err:.3e} (bound {TOL[wl.kv]})", flush=True)
    assert np.all(np.isfinite(out))
    assert err <= TOL[wl.kv]
