"""f32 activations (needs an MI355X): q, the new token's K/V and the output
in f32, over an f32 pool and over an FP8 pool.

Both the append fused into pa_decode_step and pa_kv_append followed by
pa_decode are run.  Over an FP8 pool the new token is quantised from f32 (the product with the
inverse scale taken in f32, then rounded to E4M3), so the pool after the
step is compared bit-exactly with the CPU reference's; every output element
meets the pool dtype's bound.  Query heads that share a KV head are decoded
head by head here (the matrix-core kernel takes f16 activations), so these
cases also put GQA and MQA shapes through the per-head kernel."""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_375_amd import api
from paged_kv_cache_375_amd.workloads import Workload
from tests.gpu_helpers import TOL, build_pair, out_f64, pool_bytes
from tests.test_oracle_formats import f32_store_inputs

pytestmark = pytest.mark.gpu

CASES = [
    Workload("f32act_fp8_mha_d128", 8, 8, 128, 16, 5, 1, 1300, act="f32", kv="e4m3"),
    Workload("f32act_fp8_gqa_d64", 16, 2, 64, 8, 4, 1, 1300, act="f32", kv="e4m3"),
    Workload("f32act_fp8_mqa_d32_bs1", 7, 1, 32, 1, 3, 1, 700, act="f32", kv="e4m3"),
    Workload("f32act_f32_gqa_d32", 12, 4, 32, 4, 3, 1, 900, act="f32", kv="f32"),
    Workload("f32act_f32_mha_d128_bs64", 4, 4, 128, 64, 3, 500, 1100, act="f32", kv="f32"),
]


@pytest.mark.parametrize("fused", [True, False], ids=["decode_step", "append_then_decode"])
@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_f32_activation_parity(wl, fused):
    print(f"[f32act] {wl} fused={fused}", flush=True)
    dr, gpu, ref = build_pair(wl)
    out = out_f64(gpu.run(fused=fused))
    ref.append()
    assert np.array_equal(pool_bytes(gpu.cache.k), ref.k.view(np.uint8))
    assert np.array_equal(pool_bytes(gpu.cache.v), ref.v.view(np.uint8))
    err = float(np.max(np.abs(out - ref.decode_threaded())))
    print(f"[f32act] {wl.name}: max abs err {err:.3e} (bound {TOL[wl.kv]})", flush=True)
    assert np.all(np.isfinite(out))
    assert err <= TOL[wl.kv]


@pytest.mark.parametrize("scale", [1.0, 0.012345678])
def test_fp8_store_from_f32_inputs(scale):
    """binary32 inputs at every E4M3 rounding boundary (one ulp either side),
    the saturation edge, infinities, NaN, zeros, subnormals and random bit
    patterns, stored through pa_kv_append into an E4M3 pool: byte for byte
    the reference quantiser's."""
    x = f32_store_inputs(np.random.default_rng(7))
    with np.errstate(over="ignore", invalid="ignore"):
        x = (x * np.float32(scale)).astype(np.float32)
    n = (x.size + 127) // 128
    x = np.concatenate([x, np.zeros(n * 128 - x.size, np.float32)]).reshape(n, 1, 128)
    tables = np.arange(n, dtype=np.int32).reshape(n, 1)
    ctx = np.ones(n, dtype=np.int32)
    s = np.float32(scale)
    inv = np.float32(1.0 / np.float64(s))
    cache = api.KVCache(n, 1, 1, 128, "e4m3", "cuda", float(s), float(s), float(inv), float(inv))
    xt = torch.from_numpy(x).cuda()
    api.kv_append(cache, xt, xt, torch.from_numpy(tables).cuda(), torch.from_numpy(ctx).cuda())
    got = pool_bytes(cache.k).reshape(-1)
    kp = np.zeros((n, 1, 1, 128), np.uint8)
    vp = np.zeros_like(kp)
    oracle.append(kp, vp, x, x, tables, ctx, 1, float(inv), float(inv))
    want = kp.reshape(-1)
    bad = np.nonzero(got != want)[0]
    print(f"[fp8 f32] scale {scale}: {x.size} inputs, {len(bad)} mismatches; first: "
          f"{[(hex(int(x.reshape(-1).view(np.uint32)[i])), int(got[i]), int(want[i])) for i in bad[:4]]}", flush=True)
    assert np.array_equal(got, want)
    assert np.array_equal(pool_bytes(cache.v).reshape(-1), want)
