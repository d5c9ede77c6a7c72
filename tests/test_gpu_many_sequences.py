"""Thousands of short sequences in one step (needs an MI355X).

A busy serving step can hold thousands of sequences of a few tokens each.
The grids then run long in the sequence dimension, the grouped launcher's
units far outnumber the GPU's slots (no folded order past 256 sequences),
and almost every head is a single partition written directly.  Every output
is checked against the CPU reference and the pool after the step is
bit-exact."""
import numpy as np
import pytest

from paged_kv_cache_375_amd import api
from paged_kv_cache_375_amd.workloads import Workload
from tests.gpu_helpers import TOL, build_pair, out_f64, pool_bytes

pytestmark = pytest.mark.gpu

CASES = [
    Workload("many_mha_f16", 8, 8, 128, 16, 3000, 1, 40),            # per-head kernel
    Workload("many_gqa_f16", 16, 2, 64, 8, 3000, 1, 40),             # grouped kernel (G 8)
    Workload("many_mqa_fp8", 71, 1, 64, 16, 3000, 1, 40, kv="e4m3"),  # grouped kernel (G 71), FP8 pool
]


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_many_short_sequences(wl):
    print(f"[many] {wl}", flush=True)
    dr, gpu, ref = build_pair(wl)
    out = out_f64(gpu.run())
    ref.append()
    assert np.array_equal(pool_bytes(gpu.cache.k), ref.k.view(np.uint8))
    assert np.array_equal(pool_bytes(gpu.cache.v), ref.v.view(np.uint8))
    err = float(np.max(np.abs(out - ref.decode_threaded())))
    print(f"[many] {wl.name}: max abs err {err:.3e} (bound {TOL[wl.kv]})", flush=True)
    assert np.all(np.isfinite(out))
    assert err <= TOL[wl.kv]


def test_many_sequences_sharing_a_prefix():
    """2,000 sequences forked from one 64-token prompt, FP8 pool, one query
    head per KV head: the prefix pass inside the per-head decode's launch,
    with 125 row sets per KV head."""
    wl = Workload("many_sp_fp8", 4, 4, 128, 16, 2000, 1, 30, kv="e4m3", prefix_len=64)
    print(f"[many] {wl}", flush=True)
    dr, gpu, ref = build_pair(wl)
    if gpu.step_pairs is not None:
        api.copy_blocks(gpu.cache, gpu.step_pairs)
    shared = wl.prefix_len // wl.block_size
    out = out_f64(api.decode_shared_prefix(gpu.cache, gpu.q, gpu.tables, gpu.ctx, gpu.max_ctx, gpu.sm_scale,
                                           [0, wl.batch], [shared], k_new=gpu.k_new, v_new=gpu.v_new))
    ref.append()
    assert np.array_equal(pool_bytes(gpu.cache.k), ref.k.view(np.uint8))
    assert np.array_equal(pool_bytes(gpu.cache.v), ref.v.view(np.uint8))
    err = float(np.max(np.abs(out - ref.decode_threaded())))
    print(f"[many] {wl.name}: max abs err {err:.3e} (bound {TOL[wl.kv]})", flush=True)
    assert err <= TOL[wl.kv]
