"""pa_read_probe (needs an MI355X): the measurement-only read of the pools
runs in both modes on a workload's own pools and tables, writes nothing but
its sink (and there only the fixed value it folds against), and leaves the
pools untouched."""
import numpy as np
import pytest
import torch

from paged_kv_cache_375_amd import api
from paged_kv_cache_375_amd.workloads import Workload
from tests.gpu_helpers import build_pair, pool_bytes

pytestmark = pytest.mark.gpu

MAGIC = 0x9E3779B9


@pytest.mark.parametrize("wl", [Workload("probe_mha_f16", 4, 4, 128, 16, 3, 100, 1500),
                                Workload("probe_mqa_e4m3", 8, 1, 64, 8, 3, 700, 900, kv="e4m3")],
                         ids=lambda w: w.name)
@pytest.mark.parametrize("mode", ["paged", "linear"])
def test_read_probe_reads_and_writes_nothing(wl, mode):
    print(f"[probe] {wl.name} {mode}", flush=True)
    dr, gpu, _ = build_pair(wl)
    k0, v0 = pool_bytes(gpu.cache.k), pool_bytes(gpu.cache.v)
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    for _ in range(3):
        api.read_probe(gpu.cache, gpu.tables, gpu.ctx, gpu.max_ctx, mode, sink)
    torch.cuda.synchronize()
    s = sink.cpu().numpy().view(np.uint32)
    assert np.all((s == 0) | (s == MAGIC))
    assert np.array_equal(pool_bytes(gpu.cache.k), k0)
    assert np.array_equal(pool_bytes(gpu.cache.v), v0)
