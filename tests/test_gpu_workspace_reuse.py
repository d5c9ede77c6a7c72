"""One decode workspace reused by calls whose batch grows and shrinks (needs an
MI355X).

A serving loop sizes one workspace for its largest batch and reuses it every
step, while sequences join and leave.  The workspace begins with the arrival
counters of the grouped kernel's in-launch merge of split contexts, followed
by the partials; a call with more (sequence, head) rows than an earlier one
must still find its counters at zero, never on the earlier call's partials.
Each call is checked against the CPU reference (the first n sequences of one
step: their blocks, lengths and new tokens), with split contexts throughout.
"""
import numpy as np
import pytest
import torch

from paged_kv_cache_375_amd import api
from paged_kv_cache_375_amd.workloads import WORKLOADS, Workload
from tests.gpu_helpers import TOL, build_pair, out_f64

pytestmark = pytest.mark.gpu

CASES = [
    WORKLOADS["falcon7b_mqa"].scaled(batch=6, ctx_lo=600, ctx_hi=1700),   # grouped kernel, MQA (G 71)
    WORKLOADS["llama70b_gqa"].scaled(batch=6, ctx_lo=600, ctx_hi=2100),   # grouped kernel, GQA (G 8)
    WORKLOADS["opt13b"].scaled(batch=6, ctx_lo=600, ctx_hi=1700),         # per-head kernel + merge launch
]
BATCHES = (1, 2, 6, 1, 6)


def _first(gpu, n):
    return (gpu.q[:n].contiguous(), gpu.k_new[:n].contiguous(), gpu.v_new[:n].contiguous(),
            gpu.tables[:n].contiguous(), gpu.ctx[:n].contiguous())


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_workspace_reused_as_the_batch_grows(wl):
    print(f"[workspace] {wl}", flush=True)
    dr, gpu, ref = build_pair(wl)
    assert gpu.step_pairs is None
    ws = api.new_workspace(wl.batch, wl.num_q_heads, wl.head_dim, gpu.max_ctx)
    k0, v0 = gpu.cache.k.clone(), gpu.cache.v.clone()
    ref.append()
    want = ref.decode()
    for n in BATCHES:
        c = gpu.cache.with_pools(k0.clone(), v0.clone())
        q, kn, vn, tab, ctx = _first(gpu, n)
        out = out_f64(api.decode_step(c, q, kn, vn, tab, ctx, int(dr.ctx[:n].max()), gpu.sm_scale, workspace=ws))
        err = float(np.max(np.abs(out - want[:n])))
        print(f"[workspace] {wl.name}: batch {n}, max abs err {err:.3e}", flush=True)
        assert np.all(np.isfinite(out))
        assert err <= TOL[wl.kv]
    torch.cuda.synchronize()
    assert torch.count_nonzero(ws[:wl.batch * wl.num_q_heads * 4]) == 0  # counters back at zero


def test_shared_prefix_workspace_reused_as_the_group_grows():
    """The grouped decode after a prefix pass: one shared-prefix workspace for
    groups of 1, 4 and 2 sequences in turn."""
    wl = Workload("ws_sp_gqa", 64, 8, 128, 16, 4, 600, 1200, prefix_len=512)
    print(f"[workspace] {wl}", flush=True)
    dr, gpu, ref = build_pair(wl)
    shared = wl.prefix_len // wl.block_size
    if gpu.step_pairs is not None:
        api.copy_blocks(gpu.cache, gpu.step_pairs)
    ws = torch.zeros(api.shared_workspace_size(wl.batch, wl.num_q_heads, wl.head_dim, gpu.max_ctx, wl.prefix_len),
                     dtype=torch.uint8, device="cuda")
    k0, v0 = gpu.cache.k.clone(), gpu.cache.v.clone()
    ref.append()
    want = ref.decode()
    for n in (1, 4, 2, 4):
        c = gpu.cache.with_pools(k0.clone(), v0.clone())
        q, kn, vn, tab, ctx = _first(gpu, n)
        out = out_f64(api.decode_shared_prefix(c, q, tab, ctx, int(dr.ctx[:n].max()), gpu.sm_scale, [0, n], [shared],
                                               k_new=kn, v_new=vn, workspace=ws))
        err = float(np.max(np.abs(out - want[:n])))
        print(f"[workspace] {wl.name}: group of {n}, max abs err {err:.3e}", flush=True)
        assert err <= TOL[wl.kv]
