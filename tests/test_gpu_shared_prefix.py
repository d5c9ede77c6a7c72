"""Shared-prefix decode (pa_decode_shared_prefix) against the CPU reference
(needs an MI355X).

Sequences that fork one prompt hold its full blocks in common [F55 §常见问题];
[IPX §同一提示生成两个回答的假想例子].  The shared-prefix path reads those
blocks once per KV head for all of a group's query rows, then each sequence's
own tokens, and merges both; the output must be the same attention as over
each whole context.  Cases cover FP8 and f16 pools, MHA, GQA and MQA, head
sizes 32 to 128, block sizes 1 to 64, prefixes that end on and inside a block
(the partial block is each sequence's own copy after copy-on-write), fused
and separate append, several groups, sequences outside every group, and a
group whose claim does not hold.
"""
import numpy as np
import pytest
import torch

from paged_kv_cache_375_amd import api
from paged_kv_cache_375_amd.workloads import WORKLOADS, Workload
from tests.gpu_helpers import TOL, build_pair, full_size_check, out_f64, pool_bytes

pytestmark = pytest.mark.gpu

CASES = [
    Workload("sp_fp8_mha", 40, 40, 128, 16, 6, 1, 900, kv="e4m3", prefix_len=512),
    Workload("sp_fp8_mha_505", 40, 40, 128, 16, 6, 1, 900, kv="e4m3", prefix_len=505),
    Workload("sp_f16_gqa", 64, 8, 128, 16, 4, 1, 700, prefix_len=700),
    Workload("sp_f16_mqa", 71, 1, 64, 16, 4, 1, 600, prefix_len=300),
    Workload("sp_f16_mha_bs4", 8, 8, 64, 4, 5, 1, 800, prefix_len=257),
    Workload("sp_fp8_gqa_d32_bs1", 12, 3, 32, 1, 5, 1, 400, kv="e4m3", prefix_len=130),
    # FP8 multi-head attention runs the prefix pass inside the decode launch
    # where blocks hold a wave load's tokens and at least 16 (head sizes 64
    # and 32 here), and before it otherwise (8- and 16-token blocks below)
    Workload("sp_fp8_mha_d64_bs32", 16, 16, 64, 32, 5, 1, 700, kv="e4m3", prefix_len=320),
    Workload("sp_fp8_mha_d32_bs64", 8, 8, 32, 64, 5, 1, 900, kv="e4m3", prefix_len=640),
    Workload("sp_fp8_mha_bs8", 8, 8, 128, 8, 5, 1, 600, kv="e4m3", prefix_len=200),
    Workload("sp_fp8_mha_d32_bs16", 8, 8, 32, 16, 5, 1, 600, kv="e4m3", prefix_len=256),
]


def _shared_blocks(wl):
    return wl.prefix_len // wl.block_size


def _run(gpu, group_start, group_blocks, fused):
    if gpu.step_pairs is not None:
        api.copy_blocks(gpu.cache, gpu.step_pairs)
    if fused:
        return api.decode_shared_prefix(gpu.cache, gpu.q, gpu.tables, gpu.ctx, gpu.max_ctx, gpu.sm_scale,
                                        group_start, group_blocks, k_new=gpu.k_new, v_new=gpu.v_new)
    api.kv_append(gpu.cache, gpu.k_new, gpu.v_new, gpu.tables, gpu.ctx)
    return api.decode_shared_prefix(gpu.cache, gpu.q, gpu.tables, gpu.ctx, gpu.max_ctx, gpu.sm_scale,
                                    group_start, group_blocks)


@pytest.mark.parametrize("fused", [True, False], ids=["with_append", "after_append"])
@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_shared_prefix_parity(wl, fused):
    print(f"[shared-prefix] {wl} fused={fused}", flush=True)
    dr, gpu, ref = build_pair(wl)
    shared = _shared_blocks(wl)
    t = gpu.scenario.tables
    assert (t[:, :shared] == t[0, :shared]).all()  # the sharing the call relies on
    out = out_f64(_run(gpu, [0, wl.batch], [shared], fused))
    ref.append()
    assert np.array_equal(pool_bytes(gpu.cache.k), ref.k.view(np.uint8))
    assert np.array_equal(pool_bytes(gpu.cache.v), ref.v.view(np.uint8))
    err = float(np.max(np.abs(out - ref.decode())))
    print(f"[shared-prefix] {wl.name}: max abs err {err:.3e} (bound {TOL[wl.kv]})", flush=True)
    assert np.all(np.isfinite(out))
    assert err <= TOL[wl.kv]
    again = out_f64(_run(gpu, [0, wl.batch], [shared], fused))
    assert np.array_equal(out, again)  # deterministic; counters left at zero


def test_shared_prefix_groups_and_outsiders():
    """Groups [0, 2) sharing all 32 prefix blocks, an empty group, [2, 5)
    claiming only 20 of them; sequences 5 and 6 decode as usual."""
    wl = Workload("sp_groups", 40, 40, 128, 16, 7, 1, 700, kv="e4m3", prefix_len=512)
    dr, gpu, ref = build_pair(wl)
    out = out_f64(_run(gpu, [0, 2, 2, 5], [32, 7, 20], True))
    ref.append()
    err = float(np.max(np.abs(out - ref.decode())))
    print(f"[shared-prefix] groups: max abs err {err:.3e}", flush=True)
    assert err <= TOL["e4m3"]


@pytest.mark.parametrize("kv", ["f16", "e4m3"])
def test_shared_prefix_claim_past_a_context_gives_nan_for_that_sequence_only(kv):
    wl = Workload("sp_claim", 8, 8, 64, 16, 4, 1, 200, kv=kv, prefix_len=64)
    print(f"[shared-prefix] {wl}", flush=True)
    dr, gpu, ref = build_pair(wl)
    short = int(np.argmin(dr.ctx))
    claim = (int(dr.ctx[short]) + 15) // 16  # covers the new token's slot: not a shared range
    order = [short] + [s for s in range(wl.batch) if s != short]
    perm = torch.tensor(order).cuda()
    gpu.q, gpu.k_new, gpu.v_new = gpu.q[perm].contiguous(), gpu.k_new[perm].contiguous(), gpu.v_new[perm].contiguous()
    gpu.tables, gpu.ctx = gpu.tables[perm].contiguous(), gpu.ctx[perm].contiguous()
    out = out_f64(_run(gpu, [0, 1], [claim], True))
    ref.append()
    want = ref.decode()[order]
    assert np.isnan(out[0]).all()
    assert float(np.max(np.abs(out[1:] - want[1:]))) <= TOL[kv]


def test_full_prefix_workload_parity():
    """The FP8 prefix workload at its real size, in the launch the benchmark
    times for it (shared prefix, append fused): pool bit-exact, every output
    element within the bound; the error against the unquantised f16 result
    is printed for information."""
    wl = WORKLOADS["opt13b_fp8_prefix"]
    print(f"[shared-prefix] {wl.name}: building", flush=True)
    dr, gpu, ref = build_pair(wl)
    out = out_f64(_run(gpu, [0, wl.batch], [_shared_blocks(wl)], True))
    ref.append()
    assert np.array_equal(pool_bytes(gpu.cache.k), ref.k.view(np.uint8))
    assert np.array_equal(pool_bytes(gpu.cache.v), ref.v.view(np.uint8))
    full_size_check(wl.name + " (shared-prefix path)", wl, out, ref, dr)


def random_prefix_workload(i):
    rng = np.random.default_rng(2000 + i)
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 5, 8, 16, 40, 71]))
    if i % 6 == 0:
        g = 1  # multi-head attention: the per-head decode after the prefix pass
    d = int(rng.choice([32, 64, 128]))
    bs = int(rng.choice([1, 2, 4, 8, 16, 32, 64]))
    kv = str(rng.choice(["f16", "e4m3"]))
    hq = hkv * g
    prefix = int(rng.integers(bs, 1501))  # may end inside a block
    hi = int(rng.integers(1, 1501))
    lo = int(rng.integers(1, hi + 1))
    per_seq = hq * (prefix + (lo + hi) / 2)
    b = int(rng.integers(2, int(max(2, min(40, 2e6 // per_seq))) + 1))
    return Workload(f"sprand{i}_q{hq}_kv{hkv}_d{d}_bs{bs}_{kv}_B{b}_p{prefix}_ctx{lo}-{hi}", hq, hkv, d, bs, b, lo, hi,
                    kv=kv, prefix_len=prefix)


@pytest.mark.parametrize("i", range(12))
def test_random_shared_prefix_parity(i):
    """Seeded random shapes through pa_decode_shared_prefix (one group over
    the whole batch, sharing the prefix's whole blocks), with the append
    fused: the per-head decode beside or after the prefix pass, or the
    grouped decode after it, at block
    sizes 1 to 64 and prefixes that end on or inside a block."""
    wl = random_prefix_workload(i)
    print(f"[shared-prefix] {wl.name}", flush=True)
    dr, gpu, ref = build_pair(wl)
    shared = _shared_blocks(wl)
    t = gpu.scenario.tables
    assert (t[:, :shared] == t[0, :shared]).all()
    out = out_f64(_run(gpu, [0, wl.batch], [shared], True))
    ref.append()
    assert np.array_equal(pool_bytes(gpu.cache.k), ref.k.view(np.uint8))
    assert np.array_equal(pool_bytes(gpu.cache.v), ref.v.view(np.uint8))
    err = float(np.max(np.abs(out - ref.decode_threaded())))
    print(f"[shared-prefix] {wl.name}: max abs err {err:.3e} (bound {TOL[wl.kv]})", flush=True)
    assert np.all(np.isfinite(out))
    assert err <= TOL[wl.kv]


def random_fused_case(i):
    """FP8 multi-head attention with blocks of at least 16 tokens and at least
    one wave load's tokens: the prefix pass runs inside the per-head decode's
    launch.  Random head size, block size, head count, prefix (on or inside a
    block), lengths, up to five groups (some empty) with random claims, and
    sequences outside every group at both ends."""
    rng = np.random.default_rng(3000 + i)
    d = int(rng.choice([32, 64, 128]))
    bs = int(rng.choice([b for b in (16, 32, 64) if b >= 64 // (d // 16)]))
    h = int(rng.choice([1, 3, 8, 17, 40]))
    prefix = int(rng.integers(1, 1200 // bs + 1)) * bs + int(rng.integers(0, 2)) * int(rng.integers(1, bs))
    hi = int(rng.integers(1, 1501))
    lo = int(rng.integers(1, hi + 1))
    b = int(rng.integers(2, max(3, min(48, int(1.5e6 // (h * (prefix + (lo + hi) / 2))))) + 1))
    wl = Workload(f"spfused{i}_h{h}_d{d}_bs{bs}_B{b}_p{prefix}_ctx{lo}-{hi}", h, h, d, bs, b, lo, hi, kv="e4m3",
                  prefix_len=prefix)
    k = int(rng.integers(1, 6))
    starts = sorted(int(x) for x in rng.integers(0, b + 1, size=k + 1))
    claims = [int(rng.integers(0, prefix // bs + 1)) for _ in range(k)]
    return wl, starts, claims, bool(i % 2 == 0)


@pytest.mark.parametrize("i", range(10))
def test_random_fused_shared_prefix_parity(i):
    wl, starts, claims, fused = random_fused_case(i)
    print(f"[shared-prefix] {wl.name} groups {starts} claims {claims} fused={fused}", flush=True)
    dr, gpu, ref = build_pair(wl)
    t = gpu.scenario.tables
    for g in range(len(claims)):
        assert (t[starts[g]:starts[g + 1], :claims[g]] == t[starts[g], :claims[g]]).all()
    out = out_f64(_run(gpu, starts, claims, fused))
    ref.append()
    assert np.array_equal(pool_bytes(gpu.cache.k), ref.k.view(np.uint8))
    assert np.array_equal(pool_bytes(gpu.cache.v), ref.v.view(np.uint8))
    err = float(np.max(np.abs(out - ref.decode_threaded())))
    print(f"[shared-prefix] {wl.name}: max abs err {err:.3e} (bound {TOL[wl.kv]})", flush=True)
    assert np.all(np.isfinite(out))
    assert err <= TOL[wl.kv]
