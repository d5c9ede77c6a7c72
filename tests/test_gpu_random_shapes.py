"""Seeded random decode shapes through pa_decode_step, against the CPU
reference (needs an MI355X).

Each case draws its query and KV head counts, head_dim, block size, pool
dtype, batch and context range from a fixed seed, so the launchers'
choices (per-head or grouped kernel; four or eight waves; partition length;
folded order; per-tile or per-row addressing; merge in the launch or in a
merge launch) meet combinations that no hand-picked case names.  The pool
after the step is bit-exact and every output element meets the bound."""
import numpy as np
import pytest

from paged_kv_cache_375_amd.workloads import Workload
from tests.gpu_helpers import TOL, build_pair, out_f64, pool_bytes

pytestmark = pytest.mark.gpu

N_CASES = 24


def random_workload(i):
    rng = np.random.default_rng(1000 + i)
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 3, 5, 8, 16, 24, 40, 71]))
    d = int(rng.choice([32, 64, 128]))
    bs = int(rng.choice([1, 2, 4, 8, 16, 32, 64]))
    kv = str(rng.choice(["f16", "e4m3"]))
    hq = hkv * g
    # keep the reference's work (sequences x q heads x tokens) near 2e6
    ctx_hi = int(rng.integers(1, 3001))
    ctx_lo = int(rng.integers(1, ctx_hi + 1))
    per_seq = hq * (ctx_lo + ctx_hi) / 2
    b = int(max(1, min(300, 2e6 // max(per_seq, 1))))
    b = int(rng.integers(1, b + 1))
    return Workload(f"rand{i}_q{hq}_kv{hkv}_d{d}_bs{bs}_{kv}_B{b}_ctx{ctx_lo}-{ctx_hi}", hq, hkv, d, bs, b,
                    ctx_lo, ctx_hi, kv=kv)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_parity(i):
    wl = random_workload(i)
    print(f"[rand] {wl.name}", flush=True)
    dr, gpu, ref = build_pair(wl)
    out = out_f64(gpu.run())
    ref.append()
    assert np.array_equal(pool_bytes(gpu.cache.k), ref.k.view(np.uint8))
    assert np.array_equal(pool_bytes(gpu.cache.v), ref.v.view(np.uint8))
    want = ref.decode_threaded()
    err = float(np.max(np.abs(out - want)))
    print(f"[rand] {wl.name}: max abs err {err:.3e} (bound {TOL[wl.kv]})", flush=True)
    assert np.all(np.isfinite(out))
    assert err <= TOL[wl.kv]
